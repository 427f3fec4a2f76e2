// Kernel launchers of libmoe (internal; called by api.cpp after validation).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Entries handled by one block of the counting and scatter kernels.
constexpr int kCountChunk = 2048;
// Tokens per block of the router kernel.
constexpr int kRouteSmallBatch = 2048;  // below: 4 tokens per router workgroup, else 16

hipError_t launch_route(int dtype, const void* x, const void* w_router, const float* bias, int T, int d,
                        int E, int k, int32_t* topk_ids, float* topk_w, hipStream_t stream);

hipError_t launch_count(const int32_t* ids, int Tk, int E, int nblk, int32_t* block_counts,
                        uint32_t* block_err, int32_t* token_of, int64_t fill_rows, hipStream_t stream);

struct ScanArgs {
  int32_t* block_counts;  // [nblk][E] in: per-block counts; out: per-block base ranks
  const uint32_t* block_err;
  int nblk, E, C, BM, max_tiles;
  int32_t* counts;
  int32_t* offsets;
  int32_t* spill_counts;
  int32_t* spill_offsets;
  int32_t* tile_off;  // [2][E+1]
  int32_t* tile_map;  // [2][max_tiles][4]
  int32_t* n_tiles;   // [2]
  uint32_t* err_flags;
};
hipError_t launch_scan(const ScanArgs& a, hipStream_t stream);

// Entries up to which one 1024-thread block does the whole dispatch.
constexpr int kSmallDispatch = 16384;
// Limits of the one-wavefront dispatch (a decode step): entries, experts, rows.
constexpr int kTinyDispatchEntries = 64;
constexpr int kTinyDispatchExperts = 64;
constexpr int kTinyDispatchRows = 4096;
__host__ __device__ inline bool tiny_dispatch(int Tk, int E, int64_t rows) {
  return Tk <= kTinyDispatchEntries && E <= kTinyDispatchExperts && rows <= kTinyDispatchRows;
}

struct SmallDispatchArgs {
  const int32_t* ids;
  int Tk, k, E, C, BM, max_tiles;
  int64_t rows;  // R: every row's token_of is reset to -1 first
  int32_t* counts;
  int32_t* offsets;
  int32_t* spill_counts;
  int32_t* spill_offsets;
  int32_t* row_of;
  int32_t* token_of;
  int32_t* tile_off;
  int32_t* tile_map;
  int32_t* n_tiles;
  uint32_t* err_flags;
};
hipError_t launch_dispatch_small(const SmallDispatchArgs& a, hipStream_t stream);

// Tokens up to which a batch with router weights (E <= 64) is routed and
// dispatched by one workgroup in one launch (a.ids must be topk_ids).
constexpr int kRouteDispatchTokens = 16;
hipError_t launch_route_dispatch(int dtype, const void* x, const void* w_router, const float* bias, int T, int d,
                                 int E, int k, int32_t* topk_ids, float* topk_w, const SmallDispatchArgs& a,
                                 hipStream_t stream);

hipError_t launch_scatter(const int32_t* ids, int Tk, int k, int E, int C, int nblk,
                          const int32_t* block_base, const int32_t* offsets, const int32_t* spill_offsets,
                          int32_t* row_of, int32_t* token_of, hipStream_t stream);

hipError_t launch_gather(const void* x, const int32_t* row_of, int Tk, int k, int64_t row_bytes,
                         void* x_perm, hipStream_t stream);

// One 16-byte piece per thread: groups of 16 rows of `row_bytes` bytes into
// 1024-byte blocks (see MOE_LAYOUT_BLOCKED16).
hipError_t launch_pack_blocked16(const void* src, void* dst, int64_t groups, int64_t row_bytes, hipStream_t stream);

hipError_t launch_combine(int dtype, const void* y, const float* topk_w, const int32_t* row_of, int T,
                          int k, int d, void* out, hipStream_t stream);

struct GemmArgs {
  const void* act;           // [R][K] activation rows, or (act_rows set) the source rows they come from
  const int32_t* act_rows;   // null, or [R]: row r of the activations is row act_rows[r] of `act`
  int act_nrows;             // rows of `act` when act_rows is set
  const void* w0;            // [E][N][K]
  const void* w1;            // [E][N][K] (gate+up: the up projection), else null
  const float* s0;           // fp8 weights: [E][N] per-channel scales of w0, else null
  const float* s1;           // fp8 weights: [E][N] per-channel scales of w1, else null
  void* out;                 // [R][N]
  const int32_t* tile_off;   // [E+1] of this pass
  const int32_t* tile_map;   // [max_tiles][4] of this pass
  const int32_t* n_tiles;    // [1] of this pass
  // Both passes of the capacity mode in one launch: the overflow pass's tile
  // offsets, map and count (else null).  Each expert's overflow tiles follow
  // its first-pass tiles, so both read its weights while they are in L2.
  const int32_t* tile_off2;
  const int32_t* tile_map2;
  const int32_t* n_tiles2;
  int E, K, N;
  int max_tiles;             // tiles of the map(s) the grid must cover
  int skew_map;              // 1: uneven tile counts per expert deal chunks of units to the XCDs in turn
  int blocked16;             // 1: weights in 16-row blocked order (moe_weight_layout_t)
  int wide;                  // 1: bf16 gate+up on the 160-row map may take the two-width kernel (one pass)
  float* kpart;              // non-null: bf16 down on the 160-row map splits K in two; fp32 partial sums,
                             // plane ks of [2][R][N] (kplane floats per plane)
  size_t kplane;
  // Down GEMM of a decode batch (16-row tiles, one pass) with the combine
  // folded in: non-null comb_out makes each workgroup compute its column
  // slice of y for every tile of the map, store it, and then weight it into
  // out[t] = sum_j comb_w[t k + j] y[comb_row_of[t k + j]] for that slice.
  void* comb_out;
  const float* comb_w;
  const int32_t* comb_row_of;
  int comb_T, comb_k;
};

// y[r] = rounded(part[0][r] + part[1][r]) for every row r with token_of[r] >= 0:
// the sum of the two K ranges of the split down GEMM, added in that order.
// combine straight from the split down GEMM's fp32 planes part[2][R][d]
// (plane = R*d floats): y rows formed as launch_k_split_finish forms them are
// stored and weighted into out as launch_combine weights them.
hipError_t launch_combine_split(int dtype, const float* part, size_t plane, const float* topk_w,
                                const int32_t* row_of, int T, int k, int d, void* y, void* out, hipStream_t stream);
hipError_t launch_k_split_finish(int dtype, const float* part, size_t plane, const int32_t* token_of, int64_t rows,
                                 int N, void* y, hipStream_t stream);

// Bytes of the device scratch array of moe_forward_noalloc (MOE_NOALLOC_SCRATCH_BYTES).
constexpr size_t kNoallocScratchBytes = size_t(128) << 20;

// Device address of that array on the current device, taken once per device
// (hipGetSymbolAddress) and kept; never the array's host-side name.
hipError_t noalloc_scratch(void** out);

hipError_t launch_gemm_bf16_gateup(int BM, const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemm_bf16_down(int BM, const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemm_f32_gateup(int BM, const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemm_f32_down(int BM, const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemm_fp8w_gateup(int BM, const GemmArgs& a, hipStream_t stream);
hipError_t launch_gemm_fp8w_down(int BM, const GemmArgs& a, hipStream_t stream);

inline hipError_t launch_grouped_gemm(int dtype, bool gated, int BM, const GemmArgs& a, hipStream_t stream) {
  if (a.s0 != nullptr) return gated ? launch_gemm_fp8w_gateup(BM, a, stream) : launch_gemm_fp8w_down(BM, a, stream);
  if (dtype == 1) return gated ? launch_gemm_bf16_gateup(BM, a, stream) : launch_gemm_bf16_down(BM, a, stream);
  return gated ? launch_gemm_f32_gateup(BM, a, stream) : launch_gemm_f32_down(BM, a, stream);
}

}  // namespace moe
