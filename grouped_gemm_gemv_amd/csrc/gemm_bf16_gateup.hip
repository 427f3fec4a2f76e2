// Grouped GEMM instantiations: bf16, fused gate+up SwiGLU.
#include "grouped_gemm.hpp"

namespace moe {

hipError_t launch_gemm_bf16_gateup(int BM, const GemmArgs& a, hipStream_t stream) {
  return gemm::dispatch_bm<TBF16, true>(BM, a, stream);
}

}  // namespace moe
