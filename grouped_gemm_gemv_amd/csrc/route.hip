// Router scoring and top-k softmax routing.
//
// TritonMoE review (pith.science verdict for arXiv 2605.23911), referee
// summary: the first stage of the forward pass scores every token against
// every expert.  Reading taken: softmax over all E experts, keep the k
// largest (equal logits: lower expert index first, largest first in slot
// order), renormalise the kept probabilities to sum to one.  Since the
// softmax denominator cancels in the renormalisation, the kept weights are
// exp(l_j - l_max) / sum_{kept} exp(l_j' - l_max).
//
// One workgroup handles 16 tokens.  The 16 x E logit tile is a small NT GEMM
// on the matrix cores (experts as MFMA rows, tokens as columns).  KW
// wavefronts split K (64-byte slabs, wavefront w takes slabs w, w+KW, ...),
// each issuing all loads of U slabs before its MFMAs; the KW partial tiles
// are added in a fixed order through LDS (bitwise reproducible).  Top-k, one
// token per wavefront at a time: with E <= 64 (one expert per lane) each
// expert's rank comes from one pass over the E logits (lane reads), and the
// expert of rank j moves to lane j; past 64 experts (up to 4 per lane), k
// rounds of a wavefront-wide (value, index) argmax with cross-lane shuffles.
// Either way lane j ends with slot j.
#include <float.h>

#include "device_common.hpp"
#include "dispatch_small.hpp"
#include "launch.hpp"

namespace moe {
namespace {

// NS: 16-expert subtiles (E <= 16*NS); KW: wavefronts splitting K; U: slabs
// per wavefront per round; kTok: tokens per workgroup (at most the 16 MFMA
// columns; fewer tokens spread a small batch over more compute units, while
// a large batch is better served by 16, since every workgroup reads all of
// the router weights).
// Routing of tokens t0 .. t0 + kTok - 1 by one workgroup of 64 * KW threads
// (every thread calls it).  ids_lds, if not null, also receives the chosen
// experts, in LDS at [t - t0][j], for a kernel that dispatches next.
template <class Tr, int NS, int KW, int U, int kTok>
__device__ void route_block(const typename Tr::T* __restrict__ x, const typename Tr::T* __restrict__ wr,
                            const float* __restrict__ bias, int T, int d, int E, int k, int t0,
                            int32_t* __restrict__ topk_ids, float* __restrict__ topk_w, int32_t* ids_lds) {
  using Elt = typename Tr::T;
  constexpr int E16 = NS * 16;
  __shared__ float part[KW][E16][kTok];  // per-wavefront partial logits
  __shared__ float logit[kTok][E16];

  const int lane = threadIdx.x & 63;
  // uniform in the wavefront; saying so keeps the slab index, and with it the
  // loads' K offset, in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ntok = min(kTok, T - t0);
  const int row_bytes = d * (int)sizeof(Elt);
  const int nslab = row_bytes / 64;
  // tokens past T and experts past E read as zero (buffer bounds)
  const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<Elt*>(x + (size_t)t0 * d), (short)0, ntok * row_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t wrr =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<Elt*>(wr), (short)0, E * row_bytes, 0x00020000);
  const int xoff = (lane & 15) * row_bytes + (lane >> 4) * 16;

  f32x4_t acc[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int base = 0; base < nslab; base += KW * U) {
    uint4 xa[U];
    uint4 wa[U][NS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = min(base + u * KW + wave, nslab - 1);
      xa[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(xr, xoff, s * 64, 0));
#pragma unroll
      for (int i = 0; i < NS; ++i)
        wa[u][i] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wrr, xoff + i * 16 * row_bytes, s * 64, 0));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + u * KW + wave < nslab) {
#pragma unroll
        for (int i = 0; i < NS; ++i) acc[i] = mma16<Tr>(wa[u][i], xa[u], acc[i]);
      }
    }
  }
  // acc[i][r] = partial logit of expert 16*i + 4*(lane/16) + r for token lane%16
  // (MFMA columns past kTok hold tokens of no workgroup: their loads read zeros)
  if ((lane & 15) < kTok) {
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) part[wave][i * 16 + (lane >> 4) * 4 + r][lane & 15] = acc[i][r];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < E16 * kTok; idx += 64 * KW) {
    const int e = idx / kTok, t = idx - e * kTok;
    float v = part[0][e][t];
#pragma unroll
    for (int w = 1; w < KW; ++w) v += part[w][e][t];
    if (bias != nullptr && e < E) v += bias[e];
    logit[t][e] = v;
  }
  __syncthreads();

  // top-k: wavefront w takes tokens w, w + KW, ...
  for (int tt = wave; tt < ntok; tt += KW) {
    const int t = t0 + tt;
    float v[4];
    unsigned taken = 0;  // bit q: expert lane + 64 q is chosen or absent
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = lane + 64 * q;
      v[q] = (e < E) ? logit[tt][e] : -FLT_MAX;
      if (!(e < E)) taken |= 1u << q;
    }
    int my_id = 0;
    float my_val = 0.f;
    if (E <= 64) {
      // one expert per lane: its rank is the number of experts ahead of it
      // (larger logit, or an equal logit at a lower index); the expert of
      // rank j is sent to lane j, which then holds slot j as below
      int rank = 0;
      for (int f = 0; f < E; ++f) {
        const float vf = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v[0]), f));
        rank += (vf > v[0] || (vf == v[0] && f < lane)) ? 1 : 0;
      }
      const int dst = (lane < E ? rank : lane) * 4;  // a permutation of the 64 lanes
      my_val = __builtin_bit_cast(float, __builtin_amdgcn_ds_permute(dst, __builtin_bit_cast(int, v[0])));
      my_id = __builtin_amdgcn_ds_permute(dst, lane);
    }
    for (int j = 0; j < (E <= 64 ? 0 : k); ++j) {
      float bv = -FLT_MAX;
      int bi = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        if (!((taken >> q) & 1u) && (bi == 0x7fffffff || v[q] > bv)) {
          bv = v[q];
          bi = e;
        }
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ov = __shfl_xor(bv, o);
        const int oi = __shfl_xor(bi, o);
        if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) {
          bv = ov;
          bi = oi;
        }
      }
      if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
      if (lane == j) {
        my_id = bi;
        my_val = bv;
      }
    }
    const float vmax = __shfl(my_val, 0);
    float ex = (lane < k) ? expf(my_val - vmax) : 0.f;
    float sum = ex;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane < k) {
      topk_ids[(size_t)t * k + lane] = my_id;
      topk_w[(size_t)t * k + lane] = ex / sum;
      if (ids_lds != nullptr) ids_lds[tt * k + lane] = my_id;
    }
  }
}

template <class Tr, int NS, int KW, int U, int kTok>
__global__ __launch_bounds__(64 * KW) void route_kernel(const typename Tr::T* __restrict__ x,
                                                        const typename Tr::T* __restrict__ wr,
                                                        const float* __restrict__ bias, int T, int d, int E,
                                                        int k, int32_t* __restrict__ topk_ids,
                                                        float* __restrict__ topk_w) {
  route_block<Tr, NS, KW, U, kTok>(x, wr, bias, T, d, E, k, (int)blockIdx.x * kTok, topk_ids, topk_w, nullptr);
}

// A decode batch (T <= kRouteDispatchTokens, E <= 64) routed and dispatched
// by one workgroup: the chosen experts pass to the dispatch in LDS, with no
// second launch and no round trip through global memory.
template <class Tr, int NS, int U>
__global__ __launch_bounds__(1024) void route_dispatch_kernel(const typename Tr::T* __restrict__ x,
                                                              const typename Tr::T* __restrict__ wr,
                                                              const float* __restrict__ bias, int T, int d,
                                                              int E, int k, int32_t* __restrict__ topk_ids,
                                                              float* __restrict__ topk_w, SmallDispatchArgs a) {
  __shared__ int32_t ids[kRouteDispatchTokens * 64];
  route_block<Tr, NS, 16, U, kRouteDispatchTokens>(x, wr, bias, T, d, E, k, 0, topk_ids, topk_w, ids);
  __syncthreads();
  if (tiny_dispatch(a.Tk, a.E, a.rows)) {
    if (threadIdx.x < 64) dispatch_wave(a, ids);
  } else {
    dispatch_block(a, ids);
  }
}

template <class Tr, int kTok>
hipError_t launch_t(const void* x, const void* w_router, const float* bias, int T, int d, int E, int k,
                    int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  using Elt = typename Tr::T;
  const dim3 grid((T + kTok - 1) / kTok);
  const Elt* xp = static_cast<const Elt*>(x);
  const Elt* wp = static_cast<const Elt*>(w_router);
  if (E <= 16)
    hipLaunchKernelGGL((route_kernel<Tr, 1, 16, 8, kTok>), grid, dim3(1024), 0, stream, xp, wp, bias, T, d, E, k, topk_ids, topk_w);
  else if (E <= 32)
    hipLaunchKernelGGL((route_kernel<Tr, 2, 16, 8, kTok>), grid, dim3(1024), 0, stream, xp, wp, bias, T, d, E, k, topk_ids, topk_w);
  else if (E <= 64)
    hipLaunchKernelGGL((route_kernel<Tr, 4, 16, 4, kTok>), grid, dim3(1024), 0, stream, xp, wp, bias, T, d, E, k, topk_ids, topk_w);
  else if (E <= 128)
    hipLaunchKernelGGL((route_kernel<Tr, 8, 8, 2, kTok>), grid, dim3(512), 0, stream, xp, wp, bias, T, d, E, k, topk_ids, topk_w);
  else
    hipLaunchKernelGGL((route_kernel<Tr, 16, 4, 2, kTok>), grid, dim3(256), 0, stream, xp, wp, bias, T, d, E, k, topk_ids, topk_w);
  return hipGetLastError();
}

template <class Tr>
hipError_t launch_rd(const void* x, const void* w_router, const float* bias, int T, int d, int E, int k,
                     int32_t* topk_ids, float* topk_w, const SmallDispatchArgs& a, hipStream_t stream) {
  using Elt = typename Tr::T;
  const Elt* xp = static_cast<const Elt*>(x);
  const Elt* wp = static_cast<const Elt*>(w_router);
  if (E <= 16)
    hipLaunchKernelGGL((route_dispatch_kernel<Tr, 1, 8>), dim3(1), dim3(1024), 0, stream, xp, wp, bias, T, d, E, k,
                       topk_ids, topk_w, a);
  else if (E <= 32)
    hipLaunchKernelGGL((route_dispatch_kernel<Tr, 2, 8>), dim3(1), dim3(1024), 0, stream, xp, wp, bias, T, d, E, k,
                       topk_ids, topk_w, a);
  else
    hipLaunchKernelGGL((route_dispatch_kernel<Tr, 4, 4>), dim3(1), dim3(1024), 0, stream, xp, wp, bias, T, d, E, k,
                       topk_ids, topk_w, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_dispatch(int dtype, const void* x, const void* w_router, const float* bias, int T, int d,
                                 int E, int k, int32_t* topk_ids, float* topk_w, const SmallDispatchArgs& a,
                                 hipStream_t stream) {
  if (T < 1 || T > kRouteDispatchTokens || E > 64 || a.ids != topk_ids || a.Tk != T * k)
    return hipErrorInvalidValue;
  if (dtype == 1) return launch_rd<TBF16>(x, w_router, bias, T, d, E, k, topk_ids, topk_w, a, stream);
  return launch_rd<TF32>(x, w_router, bias, T, d, E, k, topk_ids, topk_w, a, stream);
}

hipError_t launch_route(int dtype, const void* x, const void* w_router, const float* bias, int T, int d,
                        int E, int k, int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  // measured: 4 tokens per workgroup up to 2047 tokens (8.2 vs 10.2 us at
  // T = 512), 16 beyond (10.8 vs 21.7 us at T = 4096)
  if (T < kRouteSmallBatch) {
    if (dtype == 1) return launch_t<TBF16, 4>(x, w_router, bias, T, d, E, k, topk_ids, topk_w, stream);
    return launch_t<TF32, 4>(x, w_router, bias, T, d, E, k, topk_ids, topk_w, stream);
  }
  if (dtype == 1) return launch_t<TBF16, 16>(x, w_router, bias, T, d, E, k, topk_ids, topk_w, stream);
  return launch_t<TF32, 16>(x, w_router, bias, T, d, E, k, topk_ids, topk_w, stream);
}

}  // namespace moe
