// Tile shapes of the grouped GEMMs, per maximum row-tile height BM.
//
// WTN: weight rows per wavefront (per projection); WN x WK wavefronts per
// workgroup (WN split the weight rows, WK split K); PF: iterations of weight
// prefetch held in registers.  Small BM (decode-sized batches) splits K
// inside the workgroup so that narrow column tiles still give every CU work
// and enough bytes in flight; large BM gives each wavefront all rows of the
// tile so every weight byte feeds BM/16 MFMAs straight from registers.
//
// NTMS: a workgroup whose expert has a single row tile (no other workgroup
// reads its weights) loads them non-temporally if its tile has at most NTMS
// 16-row subtiles.  Measured on the Mixtral shape: 8-10 % less time per layer
// for decode batches (T = 1..128) and 5 % less for the down GEMM at T = 512;
// gate+up tiles past 4 subtiles ran 1-2 % slower with it, so they keep the
// default policy.  Experts with several row tiles keep it too, since their
// tiles share each weight byte through L2.
#pragma once

namespace moe {

template <int BM_, int WTN_, int WN_, int WK_, int PF_, int NTMS_ = 0, int RS_ = 1, int WS_ = 0, int PP_ = 0>
struct TileShape {
  static constexpr int BM = BM_, WTN = WTN_, WN = WN_, WK = WK_, PF = PF_;
  // A workgroup computes BM rows; a tile of the tile map (RS * BM rows) is
  // split into RS such pieces, so the two GEMMs can work the same tile map
  // in pieces of different heights.
  static constexpr int RS = RS_;
  // register sets of the weight prefetch: 0 = PF + 1; or PF, where the set an
  // iteration has just multiplied is refilled at once and each activation
  // fragment is read from LDS just before its MFMAs (fewer registers, the
  // same prefetch distance; the main loop unrolls PF * (PF + 1) iterations)
  static constexpr int WS = WS_;
  // tiles of at most NTMS 16-row subtiles whose expert has one row tile load
  // the weights non-temporally
  static constexpr int NTMS = NTMS_;
  // 1: the ping-pong main loop (the two wavefronts of each SIMD take turns at
  // its matrix core, one phase apart; PF weight register sets and LDS stages)
  static constexpr int PP = PP_;
};

// WQ: E4M3 weight codes; they take the bf16 shapes unless specialised below.
template <int BM, bool GATED, bool WQ = false>
struct TileCfg;
template <int BM, bool GATED>
struct TileCfg<BM, GATED, true> : TileCfg<BM, GATED, false> {};

// gate+up (two projections per wavefront).  BM 16 (a token or two per
// expert): 16 weight rows per wavefront give twice the workgroups of 32, which
// evens out the last wave of units (decode T = 1: 148 vs 154 us per layer).
template <> struct TileCfg<16, true> { using type = TileShape<16, 16, 1, 4, 4, 1>; };
template <> struct TileCfg<32, true> { using type = TileShape<32, 32, 1, 4, 4, 2>; };
template <> struct TileCfg<48, true> { using type = TileShape<48, 16, 4, 2, 4, 3>; };
template <> struct TileCfg<64, true> { using type = TileShape<64, 16, 4, 2, 4, 4>; };
template <> struct TileCfg<96, true> { using type = TileShape<96, 16, 8, 1, 4, 4>; };
template <> struct TileCfg<128, true> { using type = TileShape<128, 16, 8, 1, 4, 4>; };
template <> struct TileCfg<160, true> { using type = TileShape<160, 16, 7, 1, 4, 4>; };
template <> struct TileCfg<192, true> { using type = TileShape<192, 16, 8, 1, 3, 4, 1, 0, 1>; };
// E4M3 gate+up at BM 160 (T = 512 at the Mixtral shape): the matrix cores,
// not HBM, set its time, and with half the weight registers of bf16 the
// 32-row shape fits at 160 rows in the register-lean form; each activation
// fragment then feeds four MFMAs instead of two (gate+up 244 vs 273 us).
template <> struct TileCfg<160, true, true> { using type = TileShape<160, 32, 8, 1, 2, 4, 1, 2>; };
// BM 384 (compute-heavy shapes): the 384-row tiles of the tile map are worked
// in three 128-row pieces with 32 weight rows per wavefront, so each
// activation fragment read from LDS feeds four MFMAs (two at BM 192).
// BM 192 and 384 take the ping-pong main loop: measured against the shared
// loop, gate+up 1605 vs 1718 us at T = 4096 (Mixtral shape) and 311 vs 343
// us in the capacity workload at Gini 0.10; unchanged on the 64-expert shape.
// At BM 192 prefetch depth 3 (3 weight register sets and LDS stages in the
// ping-pong loop) against 4: capacity Gini 0.10 / 0.30 302 / 321 vs 311 /
// 332 us, 64 experts at Zipf 0 / 2.0 397 / 429 vs 404 / 436 us; depth 2 no
// faster than 4.
template <> struct TileCfg<384, true> { using type = TileShape<128, 32, 8, 1, 2, 4, 3, 0, 1>; };

// bf16 gate+up on the 160-row tile map, from about 48 rows per expert (one
// launch of grouped_gemm_wide_kernel): tiles of at most 144 rows in 224-column
// workgroups, 32 weight rows per wavefront, non-temporal weights for an
// expert with a single tile; tiles past 144 rows (whose accumulators would not
// fit in the registers at 32 weight rows per wavefront) in the 112-column
// shape above.  Measured on the vector memory path of the compute units, the
// shared limit here: each activation byte moved into LDS feeds twice the
// weight bytes (Mixtral shape, 128 rows per expert: gate+up 321 vs 363 us;
// at 32 rows per expert 2 % slower, hence the threshold).
struct Wide160 {
  using wide = TileShape<144, 32, 7, 1, 2, 9>;
  using narrow = TileCfg<160, true>::type;
};

// down projection
template <> struct TileCfg<16, false> { using type = TileShape<16, 16, 1, 4, 4, 1>; };
template <> struct TileCfg<32, false> { using type = TileShape<32, 32, 1, 4, 4, 2>; };
template <> struct TileCfg<48, false> { using type = TileShape<48, 16, 4, 2, 4, 3>; };
template <> struct TileCfg<64, false> { using type = TileShape<64, 16, 4, 2, 4, 4>; };
template <> struct TileCfg<96, false> { using type = TileShape<96, 16, 8, 1, 4, 6>; };
template <> struct TileCfg<128, false> { using type = TileShape<128, 16, 8, 1, 4, 8>; };
template <> struct TileCfg<160, false> { using type = TileShape<160, 16, 8, 1, 4, 10>; };
// BM 192 (experts past 160 rows, or the 64-expert shapes): 32 output columns
// per wavefront halve the activation reads from LDS per MFMA, which bound the
// down GEMM once tiles are tall (measured: 16-20 % faster at the capacity and
// T = 4096 workloads); prefetch depth 2 is enough there.  Non-temporal weight
// loads only up to 4 subtiles: on the 64-expert shapes that ran 1-3 % faster
// than with every single-tile expert non-temporal.
template <> struct TileCfg<192, false> { using type = TileShape<192, 32, 8, 1, 2, 4>; };
// E4M3 down at BM 160: 32 output columns per wavefront over 4 wavefronts
// (one per SIMD, so the registers suffice without the lean form); the same
// 128 columns per workgroup, half the LDS reads per MFMA (T = 512: 154 vs
// 159 us; decode T = 256: 93 vs 102 us).
template <> struct TileCfg<160, false, true> { using type = TileShape<160, 32, 4, 1, 4, 10>; };
// bf16 down (bf16 or E4M3 weights) on the 160-row tile map with many rows per expert: 256 output
// columns per workgroup (32 per wavefront) with the K loop split in two
// ranges worked by two workgroups (KS = 2 in grouped_gemm_kernel), so the
// workgroup count stays that of 128-column tiles while each activation byte
// moved into LDS feeds twice the weight bytes.
using Split160 = TileShape<160, 32, 8, 1, 4, 10>;

// BM 384: two 192-row pieces, the BM 192 shape, with the ping-pong main loop
// and prefetch depth 3 (T = 4096: down 793 vs 846 us with depth 2, 772 vs
// 809 us for depth 3 against 2).  The 192-row tiles of the map itself keep
// the shared loop: with the ping-pong loop they ran 1-3 % slower where
// experts hold 70-400 rows (64-expert and capacity workloads).
template <> struct TileCfg<384, false> { using type = TileShape<192, 32, 8, 1, 3, 4, 2, 0, 1>; };

}  // namespace moe
