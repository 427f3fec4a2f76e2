// Measurement probes of libmoe_peaks: achievable HBM streaming rates and
// bf16 matrix-core throughput on gfx950.  Self-contained (nothing shared
// with the layer's kernels); every probe leaves a result the caller checks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "moe_peaks.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 1024;    // bytes one wavefront instruction moves
constexpr int kReadWaves = 8;   // wavefronts per workgroup (read / copy)
constexpr int kMfmaChains = 8;  // independent accumulators per wavefront

// Chunk order of the read and copy probes, for wavefront gw of nw:
//  - strided (flags bit 1 clear): chunks gw, gw + nw, gw + 2 nw, ...;
//  - regions (flags bit 1 set): the contiguous chunks [gw * per, gw * per +
//    per), per = nch / nw, then chunk nw * per + gw if it exists.
// Either way every chunk is moved by exactly one wavefront, in rounds of PF
// chunks whose loads are all issued before any is used.  NT (flags bit 0):
// loads (and the copy's stores) carry the non-temporal cache policy.
template <bool NT>
__device__ __forceinline__ u32x4 ld(const char* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  else
    return *reinterpret_cast<const u32x4*>(p);
}
template <bool NT>
__device__ __forceinline__ void st(char* p, u32x4 v) {
  if constexpr (NT)
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else
    *reinterpret_cast<u32x4*>(p) = v;
}

// Calls f(c, step, N) to move chunks c, c + step, ..., c + (N-1) step of
// this wavefront: N = PF for the whole rounds, then N = 1 for the chunks
// left over.
template <bool REGION, int PF, class F>
__device__ __forceinline__ void for_chunks(size_t nch, F&& f) {
  const size_t nw = (size_t)gridDim.x * kReadWaves;
  const size_t gw = (size_t)blockIdx.x * kReadWaves + (threadIdx.x >> 6);
  if constexpr (REGION) {
    const size_t per = nch / nw;
    const size_t c0 = gw * per, c1 = c0 + per;
    size_t c = c0;
    for (; c + PF <= c1; c += PF) f(c, size_t(1), std::integral_constant<int, PF>{});
    for (; c < c1; ++c) f(c, size_t(1), std::integral_constant<int, 1>{});
    if (nw * per + gw < nch) f(nw * per + gw, size_t(1), std::integral_constant<int, 1>{});
  } else {
    size_t c = gw;
    for (; c + (PF - 1) * nw < nch; c += nw * PF) f(c, nw, std::integral_constant<int, PF>{});
    for (; c < nch; c += nw) f(c, nw, std::integral_constant<int, 1>{});
  }
}

template <bool NT, bool REGION>
__global__ __launch_bounds__(64 * kReadWaves) void read_kernel(const char* __restrict__ buf, size_t nch,
                                                               uint32_t* __restrict__ sink) {
  constexpr int PF = REGION ? 16 : 8;
  const int lane = threadIdx.x & 63;
  const char* p0 = buf + lane * 16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for_chunks<REGION, PF>(nch, [&](size_t c, size_t step, auto n) {
    constexpr int N = decltype(n)::value;
    u32x4 q[N];
#pragma unroll
    for (int p = 0; p < N; ++p) q[p] = ld<NT>(p0 + (c + p * step) * kChunk);
#pragma unroll
    for (int p = 0; p < N; ++p) acc ^= q[p];
  });
  uint32_t v = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v ^= __shfl_xor(v, o);
  __shared__ uint32_t part[kReadWaves];
  if (lane == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t s = 0;
#pragma unroll
    for (int w = 0; w < kReadWaves; ++w) s ^= part[w];
    sink[blockIdx.x] = s;
  }
}

template <bool NT, bool REGION>
__global__ __launch_bounds__(64 * kReadWaves) void copy_kernel(const char* __restrict__ src, char* __restrict__ dst,
                                                               size_t nch) {
  constexpr int PF = REGION ? 16 : 8;
  const int lane = threadIdx.x & 63;
  const char* s0 = src + lane * 16;
  char* d0 = dst + lane * 16;
  for_chunks<REGION, PF>(nch, [&](size_t c, size_t step, auto n) {
    constexpr int N = decltype(n)::value;
    u32x4 q[N];
#pragma unroll
    for (int p = 0; p < N; ++p) q[p] = ld<NT>(s0 + (c + p * step) * kChunk);
#pragma unroll
    for (int p = 0; p < N; ++p) st<NT>(d0 + (c + p * step) * kChunk, q[p]);
  });
}

// bf16 bits of f, truncated (exact for values with at most 8 significant bits)
__device__ __forceinline__ uint32_t bf16_bits(float f) { return __float_as_uint(f) >> 16; }

// At most 256 registers per wavefront (two wavefronts per SIMD): the
// accumulators then stay in place in ordinary VGPRs from one round to the
// next (with the 512 a lone wavefront may take, the compiler moved them
// between AGPRs and VGPRs every round).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void mfma_kernel(float a, float b, int iters, float* __restrict__ sink) {
  const uint32_t pa = bf16_bits(a) * 0x10001u, pb = bf16_bits(b) * 0x10001u;
  const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{pa, pa, pa, pa});
  const bf16x8 vb = __builtin_bit_cast(bf16x8, u32x4{pb, pb, pb, pb});
  f32x4 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, vb, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) s += acc[c][0];
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

int launch_status() { return hipGetLastError() == hipSuccess ? 0 : 5; }

template <class K>
int launch_rw(int flags, K&& k) {
  switch (flags) {
    case 0: k(std::integral_constant<int, 0>{}); break;
    case 1: k(std::integral_constant<int, 1>{}); break;
    case 2: k(std::integral_constant<int, 2>{}); break;
    default: k(std::integral_constant<int, 3>{}); break;
  }
  return launch_status();
}

}  // namespace

extern "C" int moe_peak_read(const void* buf, size_t bytes, uint32_t* sink, int blocks, int flags,
                             hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || bytes == 0 || bytes % kChunk != 0 || blocks < 1 || flags < 0 ||
      flags > 3 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return 1;
  const char* b = static_cast<const char*>(buf);
  return launch_rw(flags, [&](auto f) {
    constexpr int F = decltype(f)::value;
    hipLaunchKernelGGL((read_kernel<(F & 1) != 0, (F & 2) != 0>), dim3(blocks), dim3(64 * kReadWaves), 0, stream, b,
                       bytes / kChunk, sink);
  });
}

extern "C" int moe_peak_copy(const void* src, void* dst, size_t bytes, int blocks, int flags, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || bytes == 0 || bytes % kChunk != 0 || blocks < 1 || flags < 0 ||
      flags > 3 || ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) != 0)
    return 1;
  const char* s = static_cast<const char*>(src);
  char* d = static_cast<char*>(dst);
  if (s < d + bytes && d < s + bytes) return 1;
  return launch_rw(flags, [&](auto f) {
    constexpr int F = decltype(f)::value;
    hipLaunchKernelGGL((copy_kernel<(F & 1) != 0, (F & 2) != 0>), dim3(blocks), dim3(64 * kReadWaves), 0, stream, s,
                       d, bytes / kChunk);
  });
}

extern "C" int moe_peak_mfma(float a, float b, int iters, float* sink, int blocks, hipStream_t stream) {
  if (sink == nullptr || iters < 1 || blocks < 1) return 1;
  hipLaunchKernelGGL(mfma_kernel, dim3(blocks), dim3(256), 0, stream, a, b, iters, sink);
  return launch_status();
}
