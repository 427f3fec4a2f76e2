// Grouped GEMM instantiations: bf16 activations, OCP E4M3 weights with
// per-channel scales, fused gate+up SwiGLU.
#include "grouped_gemm.hpp"

namespace moe {

hipError_t launch_gemm_fp8w_gateup(int BM, const GemmArgs& a, hipStream_t stream) {
  return gemm::dispatch_bm<TBF16, true, true>(BM, a, stream);
}

}  // namespace moe
