// Grouped GEMM instantiations: f32, fused gate+up SwiGLU.
#include "grouped_gemm.hpp"

namespace moe {

hipError_t launch_gemm_f32_gateup(int BM, const GemmArgs& a, hipStream_t stream) {
  return gemm::dispatch_bm<TF32, true>(BM, a, stream);
}

}  // namespace moe
