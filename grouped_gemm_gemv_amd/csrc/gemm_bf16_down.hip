// Grouped GEMM instantiations: bf16, down projection.
#include "grouped_gemm.hpp"

namespace moe {

hipError_t launch_gemm_bf16_down(int BM, const GemmArgs& a, hipStream_t stream) {
  return gemm::dispatch_bm<TBF16, false>(BM, a, stream);
}

}  // namespace moe

#ifdef MOE_LOOP_PHASES
// Measurement library only: copies the main-loop phase sums of the bf16
// down kernels (kPhaseSlots x 8 uint64: wait for loads, barrier, activation
// loads + MFMAs, weight loads, loop total, iterations, 16-row subtiles, 1 if
// written) to host memory dst, or with clear != 0 zeroes them.  0 on success.
extern "C" int moe_loop_phases_down(void* dst, int clear) {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(moe::gemm::g_loop_phases)) != hipSuccess) return 1;
  const size_t bytes = sizeof(unsigned long long) * 8 * moe::gemm::kPhaseSlots;
  if (clear) return hipMemset(p, 0, bytes) != hipSuccess;
  return hipMemcpy(dst, p, bytes, hipMemcpyDeviceToHost) != hipSuccess;
}
#endif
