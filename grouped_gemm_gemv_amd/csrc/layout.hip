// Expert-weight storage order for the grouped GEMMs (MOE_LAYOUT_BLOCKED16):
// the rows of each matrix in groups of 16, a group stored as consecutive
// 1024-byte blocks, block c holding bytes [64c, 64c + 64) of each of its 16
// rows in row order.  A wavefront of the GEMM reads 16 rows x 64 bytes per
// load pair, so in this order its weights are one contiguous stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "launch.hpp"

namespace moe {
namespace {

// dst piece q (16 bytes) = ((group * nblk + block) * 16 + row) * 4 + piece
__global__ __launch_bounds__(256) void pack_blocked16_kernel(const uint4* __restrict__ src, uint4* __restrict__ dst,
                                                             int64_t pieces, int64_t nblk, int64_t row_pieces) {
  for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < pieces; q += (int64_t)gridDim.x * 256) {
    const int64_t j = q & 3;
    const int64_t r = (q >> 2) & 15;
    const int64_t t = q >> 6;
    const int64_t g = t / nblk;
    const int64_t c = t - g * nblk;
    dst[q] = src[(g * 16 + r) * row_pieces + c * 4 + j];
  }
}

}  // namespace

hipError_t launch_pack_blocked16(const void* src, void* dst, int64_t groups, int64_t row_bytes, hipStream_t stream) {
  const int64_t pieces = groups * row_bytes;  // 16 rows x row_bytes / 16 per group
  const int64_t blocks = std::min<int64_t>((pieces + 255) / 256, 65536);
  hipLaunchKernelGGL(pack_blocked16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), pieces, row_bytes / 64,
                     row_bytes / 16);
  return hipGetLastError();
}

}  // namespace moe
