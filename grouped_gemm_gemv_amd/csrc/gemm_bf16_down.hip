// Grouped GEMM instantiations: bf16, down projection.
#include "grouped_gemm.hpp"

namespace moe {

hipError_t launch_gemm_bf16_down(int BM, const GemmArgs& a, hipStream_t stream) {
  return gemm::dispatch_bm<TBF16, false>(BM, a, stream);
}

}  // namespace moe
