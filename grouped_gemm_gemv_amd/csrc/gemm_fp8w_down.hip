// Grouped GEMM instantiations: bf16 activations, OCP E4M3 weights with
// per-channel scales, down projection.
#include "grouped_gemm.hpp"

namespace moe {

hipError_t launch_gemm_fp8w_down(int BM, const GemmArgs& a, hipStream_t stream) {
  return gemm::dispatch_bm<TBF16, false, true>(BM, a, stream);
}

}  // namespace moe
