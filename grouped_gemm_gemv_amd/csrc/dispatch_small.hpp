// Dispatch of a small batch in one workgroup: the count, the scans over
// experts, the capacity split, the tile map and the stable ranks (the block
// schedule and permutation of the grouped GEMMs) for T*k up to
// kSmallDispatch entries.  Used by the one-block dispatch kernel and by the
// kernel that routes a decode batch and dispatches it in the same workgroup.
#pragma once

#include "device_common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

// Exclusive scan of one int per thread over a block of NW wavefronts; every
// thread of the block must call it.  `tmp` holds NW ints of LDS.
template <int NW>
__device__ int block_exclusive_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o);
    if (lane >= o) inc += n;
  }
  if (lane == 63) tmp[wave] = inc;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int t = tmp[w];
    before += (w < wave) ? t : 0;
    total += t;
  }
  __syncthreads();
  return before + inc - v;
}

// Whole dispatch (count, scans, capacity split, tile map, stable ranks) by
// one workgroup of 1024 threads, for T*k up to kSmallDispatch: the same
// results as count + scan + scatter.  Every thread of the block calls it;
// ids (global or LDS memory) replaces a.ids, so a kernel that has just chosen
// the experts can hand them over in LDS.
__device__ void dispatch_block(const SmallDispatchArgs& a, const int32_t* ids) {
  constexpr int NW = 16;
  __shared__ int hist[256];
  __shared__ int run[256];
  __shared__ int wcnt[NW][256];
  __shared__ int tmp[NW];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int E = a.E, C = a.C, BM = a.BM;
  // every entry's expert, loaded before this block stores anything: a load
  // issued after the stores below would wait for them to complete as well
  constexpr int kPer = kSmallDispatch / 1024;
  int ev[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int f = tid + 1024 * i;
    ev[i] = f < a.Tk ? ids[f] : -1;
  }
  for (int i = tid; i < 256; i += 1024) {
    hist[i] = 0;
    run[i] = 0;
  }
  for (int i = tid; i < NW * 256; i += 1024) (&wcnt[0][0])[i] = 0;
  for (int64_t r = tid; r < a.rows; r += 1024) a.token_of[r] = -1;
  __syncthreads();
  int bad = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (tid + 1024 * i < a.Tk) {
      if ((unsigned)ev[i] < (unsigned)E)
        atomicAdd(&hist[ev[i]], 1);
      else
        bad = 1;
    }
  }
  bad = __syncthreads_or(bad);
  const bool ok = tid < E;
  const int n = ok ? hist[tid] : 0;
  int total;
  const int off = block_exclusive_scan<NW>(n, tmp, total);
  const int kept = ok ? (C > 0 ? min(n, C) : n) : 0;
  const int spill = ok ? (C > 0 ? max(n - C, 0) : 0) : 0;
  int spill_total;
  const int spill_off = block_exclusive_scan<NW>(spill, tmp, spill_total);
  if (ok) {
    a.counts[tid] = n;
    a.offsets[tid] = off;
    a.spill_counts[tid] = spill;
    a.spill_offsets[tid] = spill_off;
    hist[tid] = off;          // now: first row of expert tid (uncapped)
    run[tid] = spill_off;     // now: first overflow row of expert tid, relative to E*C
  }
  if (tid == 0) {
    a.offsets[E] = total;
    a.spill_offsets[E] = spill_total;
    a.err_flags[0] = bad ? 1u : 0u;
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int rows = (p == 0) ? kept : spill;
    const int base = (p == 0) ? (C > 0 ? tid * C : off) : E * C + spill_off;
    const int tiles = (rows + BM - 1) / BM;
    int ntiles;
    const int toff = block_exclusive_scan<NW>(tiles, tmp, ntiles);
    int32_t* tile_off = a.tile_off + p * (E + 1);
    int32_t* tile_map = a.tile_map + (size_t)p * a.max_tiles * 4;
    if (ok) tile_off[tid] = toff;
    if (tid == 0) {
      tile_off[E] = ntiles;
      a.n_tiles[p] = ntiles;
    }
    for (int i = 0; i < tiles; ++i) {
      int4 ent;
      ent.x = tid;
      ent.y = base + i * BM;
      ent.z = min(BM, rows - i * BM);
      ent.w = i;
      reinterpret_cast<int4*>(tile_map)[toff + i] = ent;
    }
  }
  // stable ranks: rounds of 1024 entries in ascending f
  __shared__ int rank_base[256];
  for (int i = tid; i < 256; i += 1024) rank_base[i] = 0;
  __syncthreads();
  const int nbits = (E <= 1) ? 0 : 32 - __clz(E - 1);
  const uint64_t lt = lanemask_lt(lane);
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int f0 = 1024 * i;
    if (f0 >= a.Tk) break;
    const int f = f0 + tid;
    const bool valid = f < a.Tk;
    const int e = valid ? ev[i] : -1;
    const bool eok = valid && (unsigned)e < (unsigned)E;
    uint64_t m = __ballot(eok);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = eok && ((e >> b) & 1);
      const uint64_t bb = __ballot(bit);
      m &= bit ? bb : ~bb;
    }
    const int lrank = __popcll(m & lt);
    if (eok && lrank == 0) wcnt[wave][e] = __popcll(m);
    __syncthreads();
    if (eok) {
      int g = rank_base[e] + lrank;
      for (int w = 0; w < wave; ++w) g += wcnt[w][e];
      int row;
      if (C > 0)
        row = (g < C) ? e * C + g : E * C + run[e] + (g - C);
      else
        row = hist[e] + g;
      a.row_of[f] = row;
      a.token_of[row] = f / a.k;
    } else if (valid) {
      a.row_of[f] = -1;
    }
    __syncthreads();
    for (int i = tid; i < E; i += 1024) {
      int sum = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        sum += wcnt[w][i];
        wcnt[w][i] = 0;
      }
      rank_base[i] += sum;
    }
    __syncthreads();
  }
}


// Exclusive prefix sum over the 64 lanes of a wavefront; total: the sum.
__device__ __forceinline__ int wave_exclusive_scan(int v, int& total) {
  const int lane = threadIdx.x & 63;
  int inc = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int n = __shfl_up(inc, o);
    if (lane >= o) inc += n;
  }
  total = __shfl(inc, 63);
  return inc - v;
}

// The same dispatch as dispatch_block by one wavefront, with no workgroup
// barrier, for a batch of at most 64 entries over at most 64 experts and at
// most kTinyDispatchRows rows (a decode step).  Lane f holds entry f, lane e
// expert e; one pass over the entries gives every expert's count and
// uncapped offset and every entry's stable rank.  Rows are written once
// each: a live row gets its token, a row no entry lands on gets -1.
__device__ void dispatch_wave(const SmallDispatchArgs& a, const int32_t* ids) {
  const int lane = threadIdx.x & 63;
  const int E = a.E, C = a.C, BM = a.BM, Tk = a.Tk;
  const int my_e = lane < Tk ? ids[lane] : -1;
  const bool my_ok = lane < Tk && (unsigned)my_e < (unsigned)E;
  const uint64_t okmask = __ballot(my_ok);
  const bool bad = __ballot(lane < Tk && !my_ok) != 0;
  int n = 0, off = 0, rank = 0;
  for (int f = 0; f < Tk; ++f) {
    if (!((okmask >> f) & 1ull)) continue;
    const int ef = __builtin_amdgcn_readlane(my_e, f);
    n += (ef == lane);
    off += (ef < lane);
    rank += (f < lane && ef == my_e);
  }
  const int total = __popcll(okmask);
  const bool ok = lane < E;
  const int kept = ok ? (C > 0 ? min(n, C) : n) : 0;
  const int spill = ok ? (C > 0 ? max(n - C, 0) : 0) : 0;
  int spill_total, nt0, nt1;
  const int spill_off = wave_exclusive_scan(spill, spill_total);
  const int tiles0 = (kept + BM - 1) / BM, tiles1 = (spill + BM - 1) / BM;
  const int toff0 = wave_exclusive_scan(tiles0, nt0);
  const int toff1 = wave_exclusive_scan(tiles1, nt1);
  if (ok) {
    a.counts[lane] = n;
    a.offsets[lane] = off;
    a.spill_counts[lane] = spill;
    a.spill_offsets[lane] = spill_off;
    a.tile_off[lane] = toff0;
    a.tile_off[E + 1 + lane] = toff1;
    const int base0 = C > 0 ? lane * C : off;
    for (int i = 0; i < tiles0; ++i)
      reinterpret_cast<int4*>(a.tile_map)[toff0 + i] = make_int4(lane, base0 + i * BM, min(BM, kept - i * BM), i);
    const int base1 = E * C + spill_off;
    for (int i = 0; i < tiles1; ++i)
      reinterpret_cast<int4*>(a.tile_map + (size_t)a.max_tiles * 4)[toff1 + i] =
          make_int4(lane, base1 + i * BM, min(BM, spill - i * BM), i);
  }
  if (lane == 0) {
    a.offsets[E] = total;
    a.spill_offsets[E] = spill_total;
    a.err_flags[0] = bad ? 1u : 0u;
    a.tile_off[E] = nt0;
    a.tile_off[E + 1 + E] = nt1;
    a.n_tiles[0] = nt0;
    a.n_tiles[1] = nt1;
  }
  // entries: row and token
  const int src = my_ok ? my_e : 0;
  const int e_off = __shfl(off, src), e_spill_off = __shfl(spill_off, src);
  if (my_ok) {
    int row;
    if (C > 0)
      row = rank < C ? my_e * C + rank : E * C + e_spill_off + (rank - C);
    else
      row = e_off + rank;
    a.row_of[lane] = row;
    a.token_of[row] = lane / a.k;
  } else if (lane < Tk) {
    a.row_of[lane] = -1;
  }
  // rows no entry lands on (disjoint from the live rows written above)
  const int fixed = C > 0 ? E * C : 0;
  for (int r0 = 0; r0 < (int)a.rows; r0 += 64) {
    const int r = r0 + lane;
    const int e = r < fixed ? r / C : 0;
    const int kept_e = __shfl(kept, e);  // every lane takes part in the shuffle
    const bool dead = r < fixed ? r - e * C >= kept_e : r - fixed >= (C > 0 ? spill_total : total);
    if (r < (int)a.rows && dead) a.token_of[r] = -1;
  }
}

}  // namespace
}  // namespace moe
