// Grouped GEMM instantiations: f32, down projection.
#include "grouped_gemm.hpp"

namespace moe {

hipError_t launch_gemm_f32_down(int BM, const GemmArgs& a, hipStream_t stream) {
  return gemm::dispatch_bm<TF32, false>(BM, a, stream);
}

}  // namespace moe
