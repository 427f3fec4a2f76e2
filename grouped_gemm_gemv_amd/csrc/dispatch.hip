// Count, exclusive scan, stable permutation, capacity split, tile map,
// gather and combine.
//
// TritonMoE review (pith.science verdict for arXiv 2605.23911), referee
// summary: tokens are permuted into expert-contiguous order before the expert
// GEMMs and unpermuted with their routing weights afterwards; the grouped
// GEMM runs over fixed-size row blocks mapped to (expert, row offset) pairs
// (Algorithm 1, section 3.2).  That paper builds the block schedule on the
// host (its Limitations (5)); here it is built on the device, so the layer
// never reads counts back.  Capacity mode follows the Cap-and-Spill critique
// (juhe.plus, section "Cap-and-Spill"): at most C rows per expert in the
// first pass, the overflow compacted into one region of max(0, T*k - C)
// rows, which always suffices, for a second pass.
//
// Kernels (all grids depend only on the shape):
//   count   : one block per 2048 entries; LDS histogram of expert ids.
//   scan    : one block; per-expert scan over blocks (stable block bases),
//             exclusive scans over experts, capacity split, tile map.
//   scatter : one block per 2048 entries; stable in-block ranks from
//             wavefront ballots (a match mask built bit by bit over the
//             expert id) plus an LDS prefix across wavefronts and rounds.
//   dispatch_small : all of the above in one 1024-thread block when T*k is
//             at most kSmallDispatch (one launch instead of three).
//   dispatch_tiny : the same by one wavefront with no barrier, for at most
//             64 entries over at most 64 experts (a decode step).
//   gather  : one wavefront per entry, 16-byte vector row copy.
//   combine : one workgroup per token, fp32 weighted sum in slot order.
//   combine_split : the same from the split down GEMM's two fp32 partial
//             planes, storing each live y row on the way.
#include "device_common.hpp"
#include "dispatch_small.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void count_kernel(const int32_t* __restrict__ ids, int Tk, int E,
                                                         int32_t* __restrict__ block_counts,
                                                         uint32_t* __restrict__ block_err,
                                                         int32_t* __restrict__ token_of, int64_t fill_rows) {
  __shared__ int hist[256];
  for (int i = threadIdx.x; i < E; i += kThreads) hist[i] = 0;
  __syncthreads();
  const int base = blockIdx.x * kCountChunk;
  const int end = min(base + kCountChunk, Tk);
  int bad = 0;
  for (int f = base + threadIdx.x; f < end; f += kThreads) {
    const int e = ids[f];
    if ((unsigned)e < (unsigned)E)
      atomicAdd(&hist[e], 1);
    else
      bad = 1;
  }
  bad = __syncthreads_or(bad);
  for (int i = threadIdx.x; i < E; i += kThreads) block_counts[(size_t)blockIdx.x * E + i] = hist[i];
  if (threadIdx.x == 0) block_err[blockIdx.x] = bad ? 1u : 0u;
  // capacity mode: mark every row unused before the scatter fills live rows
  for (int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x; r < fill_rows; r += (int64_t)gridDim.x * kThreads)
    token_of[r] = -1;
}

__global__ __launch_bounds__(kThreads) void scan_kernel(ScanArgs a) {
  __shared__ int tmp[4];
  const int e = threadIdx.x;
  const bool ok = e < a.E;
  // per-expert scan over blocks: block_counts becomes each block's base rank
  int n = 0;
  if (ok) {
    for (int b = 0; b < a.nblk; ++b) {
      const size_t i = (size_t)b * a.E + e;
      const int c = a.block_counts[i];
      a.block_counts[i] = n;
      n += c;
    }
  }
  int total;
  const int off = block_exclusive_scan<4>(ok ? n : 0, tmp, total);
  const int C = a.C;
  const int kept = ok ? (C > 0 ? min(n, C) : n) : 0;
  const int spill = ok ? (C > 0 ? max(n - C, 0) : 0) : 0;
  int spill_total;
  const int spill_off = block_exclusive_scan<4>(spill, tmp, spill_total);
  if (ok) {
    a.counts[e] = n;
    a.offsets[e] = off;
    a.spill_counts[e] = spill;
    a.spill_offsets[e] = spill_off;
  }
  if (e == 0) {
    a.offsets[a.E] = total;
    a.spill_offsets[a.E] = spill_total;
  }
  const int BM = a.BM;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int rows = (p == 0) ? kept : spill;
    const int base = (p == 0) ? (C > 0 ? e * C : off) : a.E * C + spill_off;
    const int tiles = (rows + BM - 1) / BM;
    int ntiles;
    const int toff = block_exclusive_scan<4>(tiles, tmp, ntiles);
    int32_t* tile_off = a.tile_off + p * (a.E + 1);
    int32_t* tile_map = a.tile_map + (size_t)p * a.max_tiles * 4;
    if (ok) tile_off[e] = toff;
    if (e == 0) {
      tile_off[a.E] = ntiles;
      a.n_tiles[p] = ntiles;
    }
    for (int i = 0; i < tiles; ++i) {
      int4 ent;
      ent.x = e;
      ent.y = base + i * BM;
      ent.z = min(BM, rows - i * BM);
      ent.w = i;
      reinterpret_cast<int4*>(tile_map)[toff + i] = ent;
    }
  }
  if (e == 0) {
    uint32_t f = 0;
    for (int b = 0; b < a.nblk; ++b) f |= a.block_err[b];
    a.err_flags[0] = f;
  }
}

__global__ __launch_bounds__(kThreads) void scatter_kernel(const int32_t* __restrict__ ids, int Tk, int k, int E,
                                                           int C, const int32_t* __restrict__ block_base,
                                                           const int32_t* __restrict__ offsets,
                                                           const int32_t* __restrict__ spill_offsets,
                                                           int32_t* __restrict__ row_of,
                                                           int32_t* __restrict__ token_of) {
  __shared__ int run[256];
  __shared__ int wcnt[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 256; i += kThreads) {
    run[i] = 0;
    wcnt[0][i] = wcnt[1][i] = wcnt[2][i] = wcnt[3][i] = 0;
  }
  __syncthreads();
  const int nbits = (E <= 1) ? 0 : 32 - __clz(E - 1);
  const uint64_t lt = lanemask_lt(lane);
  const int base = blockIdx.x * kCountChunk;
  for (int round = 0; round < kCountChunk / kThreads; ++round) {
    const int f = base + round * kThreads + threadIdx.x;
    const bool valid = f < Tk;
    const int e = valid ? ids[f] : -1;
    const bool ok = valid && (unsigned)e < (unsigned)E;
    uint64_t m = __ballot(ok);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = ok && ((e >> b) & 1);
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const int lrank = __popcll(m & lt);
    if (ok && lrank == 0) wcnt[wave][e] = __popcll(m);
    __syncthreads();
    if (ok) {
      int r = run[e] + lrank;
      for (int w = 0; w < wave; ++w) r += wcnt[w][e];
      const int g = block_base[(size_t)blockIdx.x * E + e] + r;
      int row;
      if (C > 0)
        row = (g < C) ? e * C + g : E * C + spill_offsets[e] + (g - C);
      else
        row = offsets[e] + g;
      row_of[f] = row;
      token_of[row] = f / k;
    } else if (valid) {
      row_of[f] = -1;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < E; i += kThreads) {
      run[i] += wcnt[0][i] + wcnt[1][i] + wcnt[2][i] + wcnt[3][i];
      wcnt[0][i] = wcnt[1][i] = wcnt[2][i] = wcnt[3][i] = 0;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kThreads) void gather_kernel(const char* __restrict__ x,
                                                          const int32_t* __restrict__ row_of, int Tk, int k,
                                                          int64_t row_bytes, char* __restrict__ x_perm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int f = blockIdx.x * 4 + wave;
  if (f >= Tk) return;
  const int row = row_of[f];
  if (row < 0) return;
  const char* src = x + (size_t)(f / k) * row_bytes;
  char* dst = x_perm + (size_t)row * row_bytes;
  int64_t off = (int64_t)lane * 16;
  for (; off + 3 * 1024 < row_bytes; off += 4 * 1024) {
    const uint4 a0 = *reinterpret_cast<const uint4*>(src + off);
    const uint4 a1 = *reinterpret_cast<const uint4*>(src + off + 1024);
    const uint4 a2 = *reinterpret_cast<const uint4*>(src + off + 2048);
    const uint4 a3 = *reinterpret_cast<const uint4*>(src + off + 3072);
    *reinterpret_cast<uint4*>(dst + off) = a0;
    *reinterpret_cast<uint4*>(dst + off + 1024) = a1;
    *reinterpret_cast<uint4*>(dst + off + 2048) = a2;
    *reinterpret_cast<uint4*>(dst + off + 3072) = a3;
  }
  for (; off < row_bytes; off += 1024) *reinterpret_cast<uint4*>(dst + off) = *reinterpret_cast<const uint4*>(src + off);
}

template <class Tr>
__global__ __launch_bounds__(kThreads) void combine_kernel(const char* __restrict__ y,
                                                           const float* __restrict__ topk_w,
                                                           const int32_t* __restrict__ row_of, int T, int k,
                                                           int d, char* __restrict__ out) {
  using Elt = typename Tr::T;
  constexpr int EPC = Tr::EPC;
  const int t = blockIdx.x;
  const size_t row_bytes = (size_t)d * sizeof(Elt);
  const int nchunk = d / EPC;
  for (int c = threadIdx.x; c < nchunk; c += kThreads) {
    float acc[EPC];
#pragma unroll
    for (int i = 0; i < EPC; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += 4) {
      uint4 ch[4];
      float wj[4];
      bool ok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u;
        const int row = (j < k) ? row_of[(size_t)t * k + j] : -1;
        ok[u] = row >= 0;
        wj[u] = ok[u] ? topk_w[(size_t)t * k + j] : 0.f;
        ch[u] = ok[u] ? *reinterpret_cast<const uint4*>(y + (size_t)row * row_bytes + (size_t)c * 16)
                      : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (ok[u]) {
          float v[EPC];
          widen<Tr>(ch[u], v);
#pragma unroll
          for (int i = 0; i < EPC; ++i) acc[i] = fmaf(wj[u], v[i], acc[i]);
        }
      }
    }
    *reinterpret_cast<uint4*>(out + (size_t)t * row_bytes + (size_t)c * 16) = narrow<Tr>(acc);
  }
}

// The layer's last step when the down GEMM split its K loop: each live row of
// y is first formed from its two fp32 partial planes exactly as
// k_split_finish forms it (one fp32 add in plane order, one rounding) and
// stored, then weighted into the token's output exactly as combine_kernel
// does.  Every live row belongs to one (token, slot), so each is written once,
// and y is not read back.
template <class Tr>
__global__ __launch_bounds__(kThreads) void combine_split_kernel(const float* __restrict__ part, size_t plane,
                                                                 const float* __restrict__ topk_w,
                                                                 const int32_t* __restrict__ row_of, int T, int k,
                                                                 int d, char* __restrict__ y, char* __restrict__ out) {
  using Elt = typename Tr::T;
  constexpr int EPC = Tr::EPC;
  const int t = blockIdx.x;
  const size_t row_bytes = (size_t)d * sizeof(Elt);
  const int nchunk = d / EPC;
  for (int c = threadIdx.x; c < nchunk; c += kThreads) {
    float acc[EPC];
#pragma unroll
    for (int i = 0; i < EPC; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < k; j0 += 4) {
      float4 p0[4][EPC / 4], p1[4][EPC / 4];
      float wj[4];
      int row[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = j0 + u;
        row[u] = (j < k) ? row_of[(size_t)t * k + j] : -1;
        wj[u] = row[u] >= 0 ? topk_w[(size_t)t * k + j] : 0.f;
        const float* a = part + (size_t)(row[u] >= 0 ? row[u] : 0) * d + (size_t)c * EPC;
#pragma unroll
        for (int q = 0; q < EPC / 4; ++q) {
          p0[u][q] = row[u] >= 0 ? *reinterpret_cast<const float4*>(a + 4 * q) : float4{0.f, 0.f, 0.f, 0.f};
          p1[u][q] = row[u] >= 0 ? *reinterpret_cast<const float4*>(a + plane + 4 * q) : float4{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (row[u] >= 0) {
          float v[EPC];
#pragma unroll
          for (int q = 0; q < EPC / 4; ++q) {
            v[4 * q] = p0[u][q].x + p1[u][q].x;
            v[4 * q + 1] = p0[u][q].y + p1[u][q].y;
            v[4 * q + 2] = p0[u][q].z + p1[u][q].z;
            v[4 * q + 3] = p0[u][q].w + p1[u][q].w;
          }
          const uint4 ch = narrow<Tr>(v);
          *reinterpret_cast<uint4*>(y + (size_t)row[u] * row_bytes + (size_t)c * 16) = ch;
          widen<Tr>(ch, v);
#pragma unroll
          for (int i = 0; i < EPC; ++i) acc[i] = fmaf(wj[u], v[i], acc[i]);
        }
      }
    }
    *reinterpret_cast<uint4*>(out + (size_t)t * row_bytes + (size_t)c * 16) = narrow<Tr>(acc);
  }
}

// Sum of the two K ranges of the split down GEMM: one wavefront per row, fp32
// planes added in plane order, one rounding to the element type.
template <class Tr>
__global__ __launch_bounds__(kThreads) void k_split_finish_kernel(const float* __restrict__ part, size_t plane,
                                                                  const int32_t* __restrict__ token_of,
                                                                  int64_t rows, int N, char* __restrict__ y) {
  using Elt = typename Tr::T;
  constexpr int EPC = Tr::EPC;
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (r >= rows || token_of[r] < 0) return;
  const float* p0 = part + (size_t)r * N;
  const float* p1 = p0 + plane;
  char* yr = y + (size_t)r * N * sizeof(Elt);
  for (int c = lane * EPC; c < N; c += 64 * EPC) {
    float v[EPC];
#pragma unroll
    for (int i = 0; i < EPC; i += 4) {
      const float4 a = *reinterpret_cast<const float4*>(p0 + c + i);
      const float4 b = *reinterpret_cast<const float4*>(p1 + c + i);
      v[i] = a.x + b.x;
      v[i + 1] = a.y + b.y;
      v[i + 2] = a.z + b.z;
      v[i + 3] = a.w + b.w;
    }
    *reinterpret_cast<uint4*>(yr + (size_t)c * sizeof(Elt)) = narrow<Tr>(v);
  }
}

__global__ __launch_bounds__(1024) void dispatch_small_kernel(SmallDispatchArgs a) { dispatch_block(a, a.ids); }

__global__ __launch_bounds__(64) void dispatch_tiny_kernel(SmallDispatchArgs a) { dispatch_wave(a, a.ids); }

}  // namespace

hipError_t launch_count(const int32_t* ids, int Tk, int E, int nblk, int32_t* block_counts,
                        uint32_t* block_err, int32_t* token_of, int64_t fill_rows, hipStream_t stream) {
  hipLaunchKernelGGL(count_kernel, dim3(nblk), dim3(kThreads), 0, stream, ids, Tk, E, block_counts, block_err,
                     token_of, fill_rows);
  return hipGetLastError();
}

hipError_t launch_scan(const ScanArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* ids, int Tk, int k, int E, int C, int nblk,
                          const int32_t* block_base, const int32_t* offsets, const int32_t* spill_offsets,
                          int32_t* row_of, int32_t* token_of, hipStream_t stream) {
  hipLaunchKernelGGL(scatter_kernel, dim3(nblk), dim3(kThreads), 0, stream, ids, Tk, k, E, C, block_base, offsets,
                     spill_offsets, row_of, token_of);
  return hipGetLastError();
}

hipError_t launch_gather(const void* x, const int32_t* row_of, int Tk, int k, int64_t row_bytes,
                         void* x_perm, hipStream_t stream) {
  hipLaunchKernelGGL(gather_kernel, dim3((Tk + 3) / 4), dim3(kThreads), 0, stream, static_cast<const char*>(x),
                     row_of, Tk, k, row_bytes, static_cast<char*>(x_perm));
  return hipGetLastError();
}

hipError_t launch_dispatch_small(const SmallDispatchArgs& a, hipStream_t stream) {
  if (tiny_dispatch(a.Tk, a.E, a.rows))
    hipLaunchKernelGGL(dispatch_tiny_kernel, dim3(1), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_k_split_finish(int dtype, const float* part, size_t plane, const int32_t* token_of, int64_t rows,
                                 int N, void* y, hipStream_t stream) {
  const dim3 grid((unsigned)((rows + kThreads / 64 - 1) / (kThreads / 64))), block(kThreads);
  if (dtype == 1)
    hipLaunchKernelGGL(k_split_finish_kernel<TBF16>, grid, block, 0, stream, part, plane, token_of, rows, N,
                       static_cast<char*>(y));
  else
    hipLaunchKernelGGL(k_split_finish_kernel<TF32>, grid, block, 0, stream, part, plane, token_of, rows, N,
                       static_cast<char*>(y));
  return hipGetLastError();
}

hipError_t launch_combine_split(int dtype, const float* part, size_t plane, const float* topk_w,
                                const int32_t* row_of, int T, int k, int d, void* y, void* out, hipStream_t stream) {
  const dim3 grid(T), block(kThreads);
  if (dtype == 1)
    hipLaunchKernelGGL(combine_split_kernel<TBF16>, grid, block, 0, stream, part, plane, topk_w, row_of, T, k, d,
                       static_cast<char*>(y), static_cast<char*>(out));
  else
    hipLaunchKernelGGL(combine_split_kernel<TF32>, grid, block, 0, stream, part, plane, topk_w, row_of, T, k, d,
                       static_cast<char*>(y), static_cast<char*>(out));
  return hipGetLastError();
}

hipError_t launch_combine(int dtype, const void* y, const float* topk_w, const int32_t* row_of, int T,
                          int k, int d, void* out, hipStream_t stream) {
  const dim3 grid(T), block(kThreads);
  if (dtype == 1)
    hipLaunchKernelGGL(combine_kernel<TBF16>, grid, block, 0, stream, static_cast<const char*>(y), topk_w, row_of, T,
                       k, d, static_cast<char*>(out));
  else
    hipLaunchKernelGGL(combine_kernel<TF32>, grid, block, 0, stream, static_cast<const char*>(y), topk_w, row_of, T,
                       k, d, static_cast<char*>(out));
  return hipGetLastError();
}

}  // namespace moe
