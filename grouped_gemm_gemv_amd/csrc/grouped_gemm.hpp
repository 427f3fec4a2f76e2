// Block-scheduled grouped GEMMs of the expert FFN on the gfx950 matrix cores
// (implementation; instantiated per element type and projection in
// gemm_<type>_<projection>.hip).
//
// TritonMoE review (pith.science verdict for arXiv 2605.23911): the expert
// GEMMs run as one grouped GEMM whose fixed-size program blocks are mapped
// to (expert, token offset) pairs (referee summary, Algorithm 1, section
// 3.2); the gate and up projections share each load of the input tile and
// SiLU(gate) * up is formed in registers, so neither projection is written
// to memory (key machinery); the down projection is a separate kernel
// (desk-editor letter).
//
// Both GEMMs are "NT": activations [rows][K] and weights [N][K] are
// K-contiguous.  A workgroup owns one (row tile, column tile) pair, taken
// from the tile map the dispatch step wrote on the device; the tile count is
// read on the device and the excess workgroups of the static grid exit at
// once.  A row tile holds up to BM rows.  The number MS of its non-empty
// 16-row MFMA subtiles selects, through a switch, a main loop compiled for
// exactly MS subtiles, so the hot loop has no per-subtile branches and
// computes no empty subtile.
//
// Workgroup = WN x WK wavefronts.  Wavefront (wn, wk) owns WTN weight rows
// (per projection) starting at wn*WTN, and the K steps s with s mod WK == wk
// (a step is 128 bytes of K).  With WK > 1 the partial tiles are added in
// the order wk = 0, 1, ... through LDS at the end (small-batch shapes, where
// splitting N alone would not give enough workgroups to fill the GPU).
//
// Data movement per iteration (WK steps):
//  - the activation tile (MS*16 rows x WK*128 bytes) goes through a ring of
//    PF+1 LDS stages, PF iterations ahead, written by LDS-direct buffer loads
//    (no register round trip); with the gather folded in, each row's source
//    is row token_of[r] of x.  Chunk c of row r sits at c ^ (r & 7) so the
//    MFMA operand reads are free of bank conflicts; rows past the tile's
//    last row read as zeros;
//  - weights are streamed by each wavefront straight into MFMA operand
//    registers, PF iterations ahead, with no LDS round trip: no weight byte
//    is shared between wavefronts, and every weight byte is read from HBM
//    once per row tile.  In the blocked 16-row storage order a wavefront's
//    weights are one contiguous stream; row-major weights are read with a
//    row stride.  E4M3 weights (WQ) load 16 codes per lane per step and are
//    widened to bf16 in registers; their channel scales multiply the fp32
//    sums in the epilogue.  When the expert has a single row tile (so no
//    other workgroup reads these weights) and the tile has at most NTMS
//    subtiles, the weight loads carry the non-temporal cache policy.
// Loads are buffer loads: one descriptor per operand (bounded by the tile's
// rows, or by N for a column tail) plus 32-bit lane offsets, and reads past
// the bound return zero.  Every iteration issues the same loads (past the
// last iteration they are clamped, and their values go unused), so the
// memory counters let loads of later iterations stay in flight while earlier
// ones are consumed.
// Weights are the MFMA "A" operand (output rows = weight rows n) and the
// activations the "B" operand (output columns = token rows m), so each lane
// ends with 4 consecutive n of one row m, stored as one 8- or 16-byte write.
//
// Workgroup order is XCD-aware: gfx950 hands consecutive workgroup ids to its
// 8 XCDs round-robin, so id b is remapped to linear unit (b mod 8) * J + b / 8
// (J = units per XCD).  Each XCD therefore walks a contiguous range of units,
// ordered expert-major, then column tile, then row tile: the row tiles that
// share one weight column tile run back to back on one XCD and share its L2,
// and the activation rows of one expert stay in that XCD's L2.  When the
// routing is skewed (a few experts hold several row tiles each), contiguous
// ranges would put a hot expert's compute-heavy units on one or two XCDs;
// the units are then dealt to the XCDs in chunks of 8 consecutive units
// (chunk c to XCD c mod 8), which spreads every expert over the chip while
// consecutive units still share an XCD.  The test uses only the tile counts
// per expert, read on the device, so every workgroup takes the same mapping.
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "gemm_tiles.hpp"
#include "launch.hpp"

namespace moe {
namespace gemm {

constexpr int kKB = 128;      // bytes of K per step
constexpr int kXcdChunk = 8;  // units per chunk of the skewed workgroup-to-XCD mapping

// Main-loop phase timing, compiled only into the measurement library
// libmoe_phases.so (MOE_LOOP_PHASES): every wavefront of a WK = 1 loop sums the
// shader-clock cycles it spends waiting for its loads, waiting at the
// workgroup barrier, issuing the activation loads and MFMAs, and issuing the
// weight loads (ping-pong loop: waits, barriers, MFMA phases, load issue and
// LDS fragment reads), and stores the sums with its loop's total and the
// loop's duration on the constant 100 MHz counter in g_loop_phases
// (slot = workgroup * wavefronts + wavefront, modulo kPhaseSlots).  In the
// product library phase_clock() is a constant and the sums fold away.
constexpr int kPhaseSlots = 1 << 17;
#ifdef MOE_LOOP_PHASES
static __device__ unsigned long long g_loop_phases[kPhaseSlots * 8];
__device__ __forceinline__ unsigned long long phase_clock() {
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t = __builtin_amdgcn_s_memtime();
  __builtin_amdgcn_sched_barrier(0);
  return t;
}
// the constant 100 MHz counter, to turn loop cycles into the shader clock rate
__device__ __forceinline__ unsigned long long phase_realtime() { return __builtin_amdgcn_s_memrealtime(); }
#else
__device__ __forceinline__ constexpr unsigned long long phase_clock() { return 0; }
__device__ __forceinline__ constexpr unsigned long long phase_realtime() { return 0; }
#endif

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1 (compile-time unroll).
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<N, I + 1>(f);
  }
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Eight OCP E4M3 codes (two dwords, code j of the pair in byte j) widened to
// the eight bf16 values of one MFMA operand.  Every E4M3 value is exactly a
// bf16 value, so the widening is exact (scale 1; the channel scale is applied
// to the fp32 result).
__device__ __forceinline__ uint4 widen_e4m3(unsigned lo, unsigned hi) {
  return uint4{__builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
               __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
               __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
               __builtin_bit_cast(unsigned, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
}

// WQ: the weights are OCP E4M3 codes with one fp32 scale per output channel
// (weight row); the activations stay bf16.
// KS: the K loop of every unit is split into KS consecutive ranges worked by
// KS workgroups (KS = 1 or 2).  With KS = 2 each workgroup stores its fp32
// partial sums, unrounded, in plane ks of a [2][R][N] buffer, and a separate
// kernel adds the two planes (k_split_finish): no workgroup waits for another.
template <class Tr, int BM, int WTN, int WN, int WK, bool GATED, int PF, int NTMS, bool WQ, int WS = 0, int KS = 1,
          int PP = 0>
struct Gemm {
  using Elt = typename Tr::T;
  static_assert(!WQ || std::is_same<Tr, TBF16>::value, "fp8 weights take bf16 activations");
  static constexpr bool WQ_ = WQ;
  static constexpr int WTN_ = WTN, WN_ = WN, WK_ = WK;
  static constexpr int NTH = 64 * WN * WK;
  static constexpr int NSUB = WTN / 16;
  static constexpr int NMAT = GATED ? 2 : 1;
  static constexpr int MSUB = BM / 16;
  static constexpr int WL = NMAT * NSUB * (WQ ? 1 : 2);  // 16-byte weight loads per lane per step
  static constexpr int KWB = WQ ? kKB / 2 : kKB;  // weight bytes per row per step (64 K elements)
  static constexpr int ROWB = WK * kKB;           // activation bytes per row per iteration
  static constexpr int CPR = ROWB / 16;           // 16-byte chunks per row per iteration
  static constexpr int BN = WN * WTN;             // output columns per workgroup
  static constexpr int NW = WN * WK;              // wavefronts per workgroup
  static constexpr int NA = PF + 1;               // activation stages in LDS
  static constexpr int NWS = WS ? WS : PF + 1;     // weight register sets
  static_assert(NWS == PF || NWS == PF + 1, "weight register sets");
  static constexpr int UNR = NWS == NA ? NA : NA * NWS;  // iterations per unrolled round
  static constexpr int STAGE = BM * ROWB;         // bytes per activation stage
  static_assert(WTN % 16 == 0 && BM % 16 == 0 && PF >= 2 && PF <= 7, "tile shape");
  static_assert(KS == 1 || (KS == 2 && WK == 1 && !GATED), "K split");

  struct Ctx {
    __amdgpu_buffer_rsrc_t act;      // activation rows of the tile (reads past its rows return 0)
    const int32_t* arow;             // null, or source row of each tile row (gather folded into the loads)
    __amdgpu_buffer_rsrc_t w[NMAT];  // this workgroup's weight rows (reads past N return 0)
    int wlane[NSUB];                 // byte offset of this lane's weight row/chunk per subtile
    int wstep, whalf;                // weight bytes between K steps / between the two halves of a step
    const float* scale[NMAT];        // fp8 weights: per-channel scales of this expert
    char* out;                       // output row0
    char* stage[NA];                 // one LDS array per activation stage
    size_t ldo;                      // output row bytes
    int ld;                          // activation/weight row bytes
    int nk, nit, rows, n0, N, wk;
    int s0;                          // first K step of this workgroup's range (K split), else 0
  };

  // LDS swizzle of the activation tile: in row r, the 16-byte chunk c of each
  // 128-byte K step is stored at chunk c ^ (r & 7).  The MFMA operand read
  // (16-byte lane reads of one chunk of 16 consecutive rows, four chunks per
  // wavefront) is then free of bank conflicts; measured on gfx950 with the
  // SQ_LDS_BANK_CONFLICT counter (padding rows by 16 bytes, or other XOR
  // patterns, gave two-way conflicts).
  __device__ __forceinline__ static int swz(int r) { return r & 7; }

  // s_waitcnt that waits until at most n vector-memory operations of this
  // wavefront are outstanding (expcnt and lgkmcnt left unconstrained).
  template <int n>
  __device__ __forceinline__ static void wait_vm() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
  }

  // Cache policy of the weight loads: kNonTemporal streams them past the
  // caches' normal replacement order.  Used only where no other workgroup
  // reads the same weights (see run_ms).
  static constexpr int kNonTemporal = 2;

  // Source and LDS offsets of this wavefront's QW LDS-direct loads of an
  // activation stage of NQ 1 KB instructions (instruction q = wave + i * NW,
  // the last ones repeating instruction NQ - 1): 16-byte slot pos = 64 q +
  // lane holds chunk g of row r (swizzled); rows past the tile's last read
  // from an offset past the buffer's bound, so they load zeros.
  template <int NQ, int QW>
  __device__ __forceinline__ static void act_plan(const Ctx& c, int wave, int lane, int (&aoff)[QW], int (&lofs)[QW]) {
#pragma unroll
    for (int i = 0; i < QW; ++i) {
      const int q = min(wave + i * NW, NQ - 1);
      const int pos = q * 64 + lane;            // 16-byte slot in the stage
      const int r = pos / CPR;
      const int pc = pos - r * CPR;
      const int g = (pc & ~7) | ((pc & 7) ^ swz(r));  // chunk of the row this slot holds
      const int src = (r < c.rows) ? (c.arow != nullptr ? c.arow[r] : r) : -1;
      aoff[i] = (src >= 0) ? src * c.ld + g * 16 : 0x7ff00000;
      lofs[i] = q * 1024;
    }
  }

  // Weight loads of iteration `it` into one register set (WL 16-byte loads per
  // lane); past the last iteration the K step is clamped and the values go
  // unused.  bf16: per subtile, the two 16-byte halves of the lane's chunk of
  // the 128-byte step; E4M3: one 16-byte load holds the lane's codes of both
  // K halves.
  template <int WAUX>
  __device__ __forceinline__ static void load_w_step(const Ctx& c, int it, uint4* dst) {
    const int s = c.s0 + min(it * WK + c.wk, c.nk - 1);
    if constexpr (WQ) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < NSUB; ++i)
          dst[m * NSUB + i] = __builtin_bit_cast(
              uint4, __builtin_amdgcn_raw_buffer_load_b128(c.w[m], c.wlane[i], s * c.wstep, WAUX));
    } else {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < NSUB; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            dst[(m * NSUB + i) * 2 + h] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(c.w[m], c.wlane[i], s * c.wstep + h * c.whalf, WAUX));
    }
  }

  // The weight loads of iteration `it` that fill half h of a register set
  // (bf16: the 16-byte pieces of K half h of every subtile; E4M3: every load
  // for h = 1, none for h = 0, since one load holds both K halves).
  template <int WAUX>
  __device__ __forceinline__ static void load_w_half(const Ctx& c, int it, uint4* dst, int h) {
    const int s = c.s0 + min(it * WK + c.wk, c.nk - 1);
    if constexpr (WQ) {
      if (h == 1) load_w_step<WAUX>(c, it, dst);
    } else {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < NSUB; ++i)
          dst[(m * NSUB + i) * 2 + h] = __builtin_bit_cast(
              uint4, __builtin_amdgcn_raw_buffer_load_b128(c.w[m], c.wlane[i], s * c.wstep + h * c.whalf, WAUX));
    }
  }

  // This wavefront's qw LDS-direct loads of the activation tile of iteration
  // `it` into stage `st` (aoff: source byte offsets, lofs: LDS offsets);
  // iterations past the last are clamped to it.  (qw is a constant at every
  // call; the loop unrolls once inlined.)
  __device__ __forceinline__ static void load_a_step(const Ctx& c, int it, char* st, const int* aoff,
                                                     const int* lofs, int qw) {
    const int itc = min(it, c.nit - 1);
#pragma unroll
    for (int i = 0; i < qw; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          c.act, (__attribute__((address_space(3))) void*)(st + lofs[i]), 16, aoff[i] + itc * ROWB + c.s0 * kKB,
          0, 0, 0);
  }

  template <int MS, int WAUX>
  __device__ __forceinline__ static void run(const Ctx& c) {
    // The activation tile of an iteration (MS*16 rows x ROWB bytes) is moved
    // by LDS-direct buffer loads: one wavefront instruction fills 1 KB of LDS
    // (lane l writes bytes 16l..16l+15).  NQ instructions per stage, spread
    // over the wavefronts, QW per wavefront (the last ones repeat the final
    // instruction so every wavefront issues the same count).
    constexpr int NQ = MS * 16 * CPR / 64;
    constexpr int QW = (NQ + NW - 1) / NW;
    constexpr int WAITN = (PF - 1) * (QW + WL);   // loads issued after iteration it's loads
    const int lane = threadIdx.x & 63;
    // uniform in the wavefront; saying so keeps the LDS offsets below in
    // scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int aoff[QW];
    int lofs[QW];
    act_plan<NQ, QW>(c, wave, lane, aoff, lofs);
    // reader: row jm*16 + lane%16; swz of that row depends on the lane only
    const int rd = (lane & 15) * ROWB + c.wk * kKB;
    const int rsw = swz(lane & 15);

    f32x4_t acc[NMAT][NSUB][MS];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < NSUB; ++i)
#pragma unroll
        for (int jm = 0; jm < MS; ++jm) acc[m][i][jm] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 wq[NWS][WL];

    auto load_w = [&](int it, uint4* dst) { load_w_step<WAUX>(c, it, dst); };
    auto load_a = [&](int it, char* st) { load_a_step(c, it, st, aoff, lofs, QW); };
    // MFMA operands of one step, half h (32 of its 64 K elements).  bf16
    // weights: lane group g = lane/16 holds elements 32h + 8g .. +7 of both
    // operands.  fp8 weights: a lane's 16 codes are elements 16g .. 16g+15,
    // so half h takes elements 16g + 8h .. +7, and the activation read follows
    // the same order (any K order shared by both operands gives the same sum).
    auto compute = [&](const char* st, const uint4* w) {
      const char* lb = st + rd;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int chunk = WQ ? 2 * (lane >> 4) + h : h * 4 + (lane >> 4);
        const int co = (chunk ^ rsw) * 16;
        uint4 wop[NMAT * NSUB];
#pragma unroll
        for (int q = 0; q < NMAT * NSUB; ++q) {
          if constexpr (WQ)
            wop[q] = h == 0 ? widen_e4m3(w[q].x, w[q].y) : widen_e4m3(w[q].z, w[q].w);
          else
            wop[q] = w[q * 2 + h];
        }
        if constexpr (NWS == PF) {
          // register-lean shapes: each activation fragment is read just
          // before its MFMAs
#pragma unroll
          for (int jm = 0; jm < MS; ++jm) {
            const uint4 a = *reinterpret_cast<const uint4*>(lb + jm * 16 * ROWB + co);
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
              for (int i = 0; i < NSUB; ++i) acc[m][i][jm] = mma16<Tr>(wop[m * NSUB + i], a, acc[m][i][jm]);
          }
        } else {
          uint4 af[MS];
#pragma unroll
          for (int jm = 0; jm < MS; ++jm) af[jm] = *reinterpret_cast<const uint4*>(lb + jm * 16 * ROWB + co);
#pragma unroll
          for (int jm = 0; jm < MS; ++jm)
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
              for (int i = 0; i < NSUB; ++i) acc[m][i][jm] = mma16<Tr>(wop[m * NSUB + i], af[jm], acc[m][i][jm]);
        }
      }
    };
    // One iteration `it` (u = it mod UNR; stage u mod NA and weight registers
    // u mod NWS, so the indices are compile-time and each LDS stage is its
    // own array: the compiler then knows loads into one stage do not alias
    // reads of another):
    //   1. wait until this wavefront's loads of iteration `it` (activation
    //      tile and weights, issued PF iterations ago) have landed; later
    //      iterations' loads stay in flight;
    //   2. barrier (without a release fence, which would drain every
    //      LDS-direct load): every wavefront's part of the tile is in LDS and
    //      every wavefront is done with stage (it - 1) mod NA;
    //   3. issue the activation tile of it + PF into that free stage;
    //   4. MFMAs of iteration `it`;
    //   5. issue the weights of it + PF into the registers freed last
    //      iteration (or, with NWS = PF, into the ones just multiplied).
    // The gate+up kernel raises the wavefront's issue priority while it issues
    // loads, so a wavefront busy with MFMAs on the same SIMD does not delay the
    // next loads (measured 1.5 % at 128 rows per expert; no gain for down).
    [[maybe_unused]] unsigned long long ph_wait = 0, ph_bar = 0, ph_mma = 0, ph_wload = 0;
    [[maybe_unused]] const unsigned long long ph_start = phase_clock(), ph_rt = phase_realtime();
    auto body = [&](int it, auto uc, auto waitc) {
      constexpr int u = decltype(uc)::value;
      const unsigned long long t0 = phase_clock();
      wait_vm<decltype(waitc)::value>();
      const unsigned long long t1 = phase_clock();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      const unsigned long long t2 = phase_clock();
      if constexpr (GATED) __builtin_amdgcn_s_setprio(2);
      load_a(it + PF, c.stage[(u + PF) % NA]);
      if constexpr (GATED) __builtin_amdgcn_s_setprio(0);
      __builtin_amdgcn_sched_barrier(0);
      if (WK == 1 || it * WK + c.wk < c.nk) compute(c.stage[u % NA], wq[u % NWS]);
      __builtin_amdgcn_sched_barrier(0);
      const unsigned long long t3 = phase_clock();
      if constexpr (GATED) __builtin_amdgcn_s_setprio(2);
      load_w(it + PF, wq[(u + PF) % NWS]);
      if constexpr (GATED) __builtin_amdgcn_s_setprio(0);
      const unsigned long long t4 = phase_clock();
      ph_wait += t1 - t0;
      ph_bar += t2 - t1;
      ph_mma += t3 - t2;
      ph_wload += t4 - t3;
    };

#pragma unroll
    for (int u = 0; u < PF; ++u) {
      load_a(u, c.stage[u]);
      load_w(u, wq[u]);
    }
    int it0 = 0;
    for (; it0 + UNR <= c.nit; it0 += UNR) {
      static_for<UNR>([&](auto uc) { body(it0 + decltype(uc)::value, uc, std::integral_constant<int, WAITN>{}); });
    }
    // The last nit mod UNR iterations.  Weight loads of the tail whose values
    // no later iteration uses may be dropped by the compiler, so tail
    // iteration u counts only what is surely issued after its own loads:
    // when those came from the loop (u < PF), all loads of the loop's last
    // PF - 1 - u iterations and the activation loads of the u tail iterations
    // before it; when they came from the tail, the activation loads of the
    // PF - 1 tail iterations in between.  (Waiting for WAITN there could let
    // a wavefront reach the barrier before its activation loads had landed.)
    static_for<UNR>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      constexpr int n = u < PF ? (PF - 1 - u) * (QW + WL) + u * QW : (PF - 1) * QW;
      if (it0 + u < c.nit) body(it0 + u, uc, std::integral_constant<int, n>{});
    });
    // the trailing (clamped) loads still write LDS: drain them before the
    // LDS is reused or the wavefront ends
    wait_vm<0>();
    __syncthreads();
#ifdef MOE_LOOP_PHASES
    if constexpr (WK == 1) {
      const unsigned slot = (blockIdx.x * NW + (threadIdx.x >> 6)) % kPhaseSlots;
      if (lane == 0) {
        unsigned long long* o = g_loop_phases + (size_t)slot * 8;
        o[0] = ph_wait;
        o[1] = ph_bar;
        o[2] = ph_mma;
        o[3] = ph_wload;
        o[4] = phase_clock() - ph_start;
        o[5] = c.nit;
        o[6] = phase_realtime() - ph_rt;
        o[7] = 1;
      }
    }
#endif


    if constexpr (WK > 1) {
      // add the partial tiles of wk = 1, 2, ... into wk = 0, in that order
      constexpr int PART = NMAT * NSUB * MS * 4 * 64;  // floats per wavefront partial
      // wavefront column wn reduces through LDS stage wn
      static_assert((size_t)PART * sizeof(float) <= (size_t)STAGE && WN <= NA, "LDS too small for split-K");
      // (select with static indices: a run-time index into c.stage would put
      // the whole context in scratch memory)
      const int wn = (threadIdx.x >> 6) % WN;
      char* redb = c.stage[0];
#pragma unroll
      for (int i = 1; i < WN; ++i)
        if (wn == i) redb = c.stage[i];
      float* red = reinterpret_cast<float*>(redb);
      for (int src = 1; src < WK; ++src) {
        if (c.wk == src) {
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int i = 0; i < NSUB; ++i)
#pragma unroll
              for (int jm = 0; jm < MS; ++jm)
#pragma unroll
                for (int r = 0; r < 4; ++r) red[(((m * NSUB + i) * MS + jm) * 4 + r) * 64 + lane] = acc[m][i][jm][r];
        }
        __syncthreads();
        if (c.wk == 0) {
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int i = 0; i < NSUB; ++i)
#pragma unroll
              for (int jm = 0; jm < MS; ++jm)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[m][i][jm][r] += red[(((m * NSUB + i) * MS + jm) * 4 + r) * 64 + lane];
        }
        __syncthreads();
      }
      if (c.wk != 0) return;
    }

    store_tile<MS>(c, acc);
  }

  // Ping-pong main loop (PP): the two wavefronts that share a SIMD (wave w
  // and w + NW/2: gfx950 places the wavefronts of a workgroup on the SIMDs
  // with period 4) take turns at its matrix core, so that one issues MFMAs
  // while the other waits for memory, issues loads and reads its next
  // operands from LDS.  Each half step (32 K elements) of an iteration is
  // one MFMA phase; phases are separated by workgroup barriers, and the
  // second group of wavefronts runs one phase behind the first.  Per
  // iteration i (stage and weight register set i mod PF), a wavefront runs
  //   MFMA(i, half 0)                       [operands already in registers]
  //   MEM0: issue iteration i + PF's weights for K half 0 (into the half of
  //         the set just multiplied); read half 1's activation fragments of
  //         stage i; wait until its own loads of iteration i + 1's
  //         activations have landed
  //   MFMA(i, half 1)
  //   MEM1: issue iteration i + PF's weights for K half 1 and its activation
  //         tile (into stage i mod PF, whose fragments every wavefront has
  //         read: each reads them before a barrier that precedes this phase,
  //         and waits for the reads); read half 0's fragments of stage i + 1
  //         (landed: every wavefront waited for its part in its MEM0 before a
  //         barrier that precedes this phase); wait until its weights of
  //         iteration i + 1 for half 0 have landed (half 1's are covered by
  //         the next MEM0's wait, since they were issued before the
  //         activations it waits for)
  // with a barrier after each of the four.  The second group adds one barrier
  // before the loop and the first one after it, so every wavefront passes
  // the same number of barriers.  Each wavefront waits for its LDS reads
  // before the barrier that ends a memory phase, so its MFMA phase needs no
  // wait.  Splitting the weight loads over both memory phases keeps each
  // phase's burst of loads (four wavefronts of a compute unit issue at once)
  // within what the compute unit's load path moves during an MFMA phase.
  // The activation fragments of one half step are the only operand registers
  // beyond the weight sets, so the tile fits in the registers of two
  // wavefronts per SIMD.
  template <int MS, int WAUX>
  __device__ __forceinline__ static void run_pp(const Ctx& c) {
    static_assert(WK == 1 && NW % 2 == 0 && PF >= 2, "ping-pong shape");
    constexpr int NQ = MS * 16 * CPR / 64;
    constexpr int QW = (NQ + NW - 1) / NW;
    // loads per iteration: W0 weight loads in MEM0 (K half 0 of the set just
    // multiplied), then W1 weight loads and the QW activation loads in MEM1
    constexpr int W0 = WQ ? 0 : WL / 2, W1 = WL - W0, L = WL + QW;
    constexpr int WAIT_A = W0 + (PF - 2) * L;       // MEM0: activations of i + 1 landed
    constexpr int WAIT_W = W1 + QW + (PF - 1) * L;  // MEM1: weights of i + 1 for half 0 landed
    constexpr int WAIT_0 = (PF - 1) * L;            // prologue: iteration 0 landed
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bool second = wave >= NW / 2;
    int aoff[QW];
    int lofs[QW];
    act_plan<NQ, QW>(c, wave, lane, aoff, lofs);
    const int rd = (lane & 15) * ROWB;
    const int rsw = swz(lane & 15);

    f32x4_t acc[NMAT][NSUB][MS];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < NSUB; ++i)
#pragma unroll
        for (int jm = 0; jm < MS; ++jm) acc[m][i][jm] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    uint4 wq[PF][WL];
    uint4 af[MS];
    auto load_w = [&](int it, uint4* dst, int h) { load_w_half<WAUX>(c, it, dst, h); };
    auto load_a = [&](int it, char* st) { load_a_step(c, it, st, aoff, lofs, QW); };

    auto barrier = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      __builtin_amdgcn_sched_barrier(0);
    };
    // activation fragments of half h from stage st (same K order as `run`)
    auto read_frags = [&](const char* st, int h) {
      const int chunk = WQ ? 2 * (lane >> 4) + h : h * 4 + (lane >> 4);
      const char* lb = st + rd + (chunk ^ rsw) * 16;
#pragma unroll
      for (int jm = 0; jm < MS; ++jm) af[jm] = *reinterpret_cast<const uint4*>(lb + jm * 16 * ROWB);
    };
    auto wait_lds = [&]() { __builtin_amdgcn_s_waitcnt((63 & 15) | ((63 >> 4) << 14) | (7 << 4) | (0 << 8)); };
    auto mfma_half = [&](const uint4* w, int h) {
      uint4 wop[NMAT * NSUB];
#pragma unroll
      for (int q = 0; q < NMAT * NSUB; ++q) {
        if constexpr (WQ)
          wop[q] = h == 0 ? widen_e4m3(w[q].x, w[q].y) : widen_e4m3(w[q].z, w[q].w);
        else
          wop[q] = w[q * 2 + h];
      }
#pragma unroll
      for (int jm = 0; jm < MS; ++jm)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int i = 0; i < NSUB; ++i) acc[m][i][jm] = mma16<Tr>(wop[m * NSUB + i], af[jm], acc[m][i][jm]);
    };
    // One iteration.  In the main loop every iteration issues the loads of
    // iteration it + PF (clamped past the last, so the counts of the waits
    // hold).  TAIL: one of the last nit mod PF iterations, which issues no
    // loads (they would be for iterations past the last); what it still has
    // to wait for was issued in the main loop, so it waits for all of that.
    // phase sums (measurement build only): waits for loads and LDS reads,
    // barriers, MFMA phases, load issue and fragment reads
    [[maybe_unused]] unsigned long long ph_wait = 0, ph_bar = 0, ph_mma = 0, ph_issue = 0;
    [[maybe_unused]] const unsigned long long ph_start = phase_clock(), ph_rt = phase_realtime();
    auto tbar = [&]() {
      const unsigned long long t = phase_clock();
      barrier();
      ph_bar += phase_clock() - t;
    };
    auto body = [&](int it, auto uc, auto tailc) {
      constexpr int u = decltype(uc)::value;
      constexpr bool TAIL = decltype(tailc)::value;
      unsigned long long t = phase_clock();
      mfma_half(wq[u], 0);
      ph_mma += phase_clock() - t;
      tbar();
      t = phase_clock();
      if constexpr (!TAIL) load_w(it + PF, wq[u], 0);
      read_frags(c.stage[u], 1);
      ph_issue += phase_clock() - t;
      t = phase_clock();
      if constexpr (TAIL) {
        if (it + 1 < c.nit) wait_vm<0>();
      } else {
        wait_vm<WAIT_A>();
      }
      wait_lds();
      ph_wait += phase_clock() - t;
      tbar();
      t = phase_clock();
      mfma_half(wq[u], 1);
      ph_mma += phase_clock() - t;
      tbar();
      t = phase_clock();
      if constexpr (!TAIL) {
        load_w(it + PF, wq[u], 1);
        load_a(it + PF, c.stage[u]);
      }
      read_frags(c.stage[(u + 1) % PF], 0);
      ph_issue += phase_clock() - t;
      t = phase_clock();
      if constexpr (TAIL) {
        if (it + 1 < c.nit) wait_vm<0>();
      } else {
        wait_vm<WAIT_W>();
      }
      wait_lds();
      ph_wait += phase_clock() - t;
      tbar();
    };

#pragma unroll
    for (int u = 0; u < PF; ++u) {
      load_w(u, wq[u], 0);
      load_w(u, wq[u], 1);
      load_a(u, c.stage[u]);
    }
    wait_vm<WAIT_0>();
    barrier();
    read_frags(c.stage[0], 0);
    wait_lds();
    if (second) barrier();
    // whole rounds of PF iterations with no run-time test inside (the wait
    // counts the compiler derives then match the explicit ones), then the
    // rest; an iteration past the last is skipped by every wavefront alike,
    // its barriers with it
    int it0 = 0;
    for (; it0 + PF <= c.nit; it0 += PF)
      static_for<PF>([&](auto uc) { body(it0 + decltype(uc)::value, uc, std::false_type{}); });
    static_for<PF - 1>([&](auto uc) {
      if (it0 + decltype(uc)::value < c.nit) body(it0 + decltype(uc)::value, uc, std::true_type{});
    });
    if (!second) barrier();
    // the trailing (clamped) loads still write LDS: drain them before the
    // LDS is reused or the wavefront ends
    wait_vm<0>();
    __syncthreads();
#ifdef MOE_LOOP_PHASES
    {
      const unsigned slot = (blockIdx.x * NW + wave) % kPhaseSlots;
      if (lane == 0) {
        unsigned long long* o = g_loop_phases + (size_t)slot * 8;
        o[0] = ph_wait;
        o[1] = ph_bar;
        o[2] = ph_mma;
        o[3] = ph_issue;
        o[4] = phase_clock() - ph_start;
        o[5] = c.nit;
        o[6] = phase_realtime() - ph_rt;
        o[7] = 1;
      }
    }
#endif
    store_tile<MS>(c, acc);
  }

  // Epilogue of a workgroup's tile: lane holds rows n = n0 + 16 i + 4 (lane/16)
  // + r of column m (fp8 weights: times the scale of channel n); gate+up
  // stores silu(gate) * up, down the sum (fp32 partial sums with the K split).
  template <int MS>
  __device__ __forceinline__ static void store_tile(const Ctx& c, const f32x4_t (&acc)[NMAT][NSUB][MS]) {
    const int lane = threadIdx.x & 63;
    float sc[NMAT][NSUB][4];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < NSUB; ++i) {
        const int n = c.n0 + i * 16 + (lane >> 4) * 4;
        float4 v4 = float4{1.f, 1.f, 1.f, 1.f};
        if constexpr (WQ) {
          if (n < c.N) v4 = *reinterpret_cast<const float4*>(c.scale[m] + n);
        }
        sc[m][i][0] = v4.x;
        sc[m][i][1] = v4.y;
        sc[m][i][2] = v4.z;
        sc[m][i][3] = v4.w;
      }
#pragma unroll
    for (int jm = 0; jm < MS; ++jm) {
      const int m = jm * 16 + (lane & 15);
      if (m < c.rows) {
        char* orow = c.out + (size_t)m * c.ldo;
#pragma unroll
        for (int i = 0; i < NSUB; ++i) {
          const int n = c.n0 + i * 16 + (lane >> 4) * 4;
          if (n < c.N) {
            float v[4];
#pragma unroll
            for (int r = 0; r < 4; ++r)
              v[r] = GATED ? silu_mul(acc[0][i][jm][r] * sc[0][i][r], acc[NMAT - 1][i][jm][r] * sc[NMAT - 1][i][r])
                           : acc[0][i][jm][r] * sc[0][i][r];
            if constexpr (KS == 2)
              store4<TF32>(orow + (size_t)n * sizeof(float), v[0], v[1], v[2], v[3]);
            else
              store4<Tr>(orow + (size_t)n * sizeof(Elt), v[0], v[1], v[2], v[3]);
          }
        }
      }
    }
  }

  // Main loop for exactly ms subtiles.  `once`: the expert has a single row
  // tile in this launch, so each weight byte is read by one workgroup only;
  // tiles of at most NTMS subtiles then load the weights non-temporally.
  template <int M, int WAUX>
  __device__ __forceinline__ static void go(const Ctx& c) {
    if constexpr (PP)
      run_pp<M, WAUX>(c);
    else
      run<M, WAUX>(c);
  }

  template <int M>
  __device__ __forceinline__ static void run_ms(int ms, bool once, const Ctx& c) {
    if constexpr (M >= 1) {
      if (ms == M) {
        if constexpr (M <= NTMS) {
          if (once) {
            go<M, kNonTemporal>(c);
            return;
          }
        }
        go<M, 0>(c);
        return;
      }
      run_ms<M - 1>(ms, once, c);
    }
  }
};

// Fill the context of one workgroup of Gemm G: expert e, tile rows
// [row0, row0 + rows), weight rows [nbase, nbase + G::BN) of each projection;
// `stages` are the workgroup's LDS stage arrays.
template <class G>
__device__ __forceinline__ void setup_ctx(typename G::Ctx& c, const GemmArgs& p, char* const* stages, int e,
                                          int row0, int rows, int nbase, int wave, int lane) {
  using Elt = typename G::Elt;
  constexpr bool WQ = G::WQ_;
  const int ld = p.K * (int)sizeof(Elt);
  c.ld = ld;
  c.ldo = (size_t)p.N * sizeof(Elt);
  c.nk = ld / kKB;
  c.nit = (c.nk + G::WK_ - 1) / G::WK_;
  c.s0 = 0;
  c.rows = rows;
  c.N = p.N;
  c.wk = wave / G::WN_;
  c.n0 = nbase + (wave % G::WN_) * G::WTN_;
  c.out = reinterpret_cast<char*>(p.out) + (size_t)row0 * c.ldo;
#pragma unroll
  for (int i = 0; i < G::NA; ++i) c.stage[i] = stages[i];
  if (p.act_rows != nullptr) {
    // activation row r of the tile is row act_rows[row0 + r] of the source
    c.arow = p.act_rows + row0;
    c.act = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.act), (short)0, p.act_nrows * ld, 0x00020000);
  } else {
    c.arow = nullptr;
    c.act = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(p.act) + (size_t)row0 * ld), (short)0, rows * ld, 0x00020000);
  }
  const int ldw = WQ ? p.K : ld;               // weight row bytes (one byte per fp8 code)
  const size_t wbase = (size_t)e * p.N * ldw + (size_t)nbase * ldw;
  const int wbytes = min(G::BN, p.N - nbase) * ldw;  // reads past N return 0 (column tail)
  c.w[0] = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(reinterpret_cast<const char*>(p.w0) + wbase),
                                             (short)0, wbytes, 0x00020000);
  if (G::NMAT == 2)
    c.w[G::NMAT - 1] = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(reinterpret_cast<const char*>(p.w1) + wbase), (short)0, wbytes, 0x00020000);
  // row-major: lane reads row (lane % 16) of the subtile, 16 bytes at
  // 16 (lane / 16) of each 64-byte half step.  Blocked 16-row order: the
  // same bytes sit at row * 64 inside the 1024-byte block of that half step.
  const int rowpitch = p.blocked16 ? 64 : ldw;
  c.wstep = p.blocked16 ? 16 * G::KWB : G::KWB;
  c.whalf = p.blocked16 ? 1024 : 64;
#pragma unroll
  for (int i = 0; i < G::NSUB; ++i)
    c.wlane[i] = ((wave % G::WN_) * G::WTN_ + 16 * i) * ldw + (lane & 15) * rowpitch + (lane >> 4) * 16;
  if constexpr (WQ) {
    c.scale[0] = p.s0 + (size_t)e * p.N;
    c.scale[G::NMAT - 1] = (G::NMAT == 2 ? p.s1 : p.s0) + (size_t)e * p.N;
  }
}

template <class Tr, int BM, int WTN, int WN, int WK, bool GATED, int PF, int NTMS, bool WQ, int RS, int WS, int KS,
          int PP>
__global__ __launch_bounds__(64 * WN * WK) void grouped_gemm_kernel(GemmArgs p) {
  using G = Gemm<Tr, BM, WTN, WN, WK, GATED, PF, NTMS, WQ, WS, KS, PP>;
  // one LDS array per activation stage (stages past NA are 16-byte stubs)
  __shared__ __attribute__((aligned(16))) char st0[G::STAGE];
  __shared__ __attribute__((aligned(16))) char st1[G::STAGE];
  __shared__ __attribute__((aligned(16))) char st2[G::STAGE];
  __shared__ __attribute__((aligned(16))) char st3[G::NA > 3 ? G::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st4[G::NA > 4 ? G::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st5[G::NA > 5 ? G::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st6[G::NA > 6 ? G::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st7[G::NA > 7 ? G::STAGE : 16];
  const int lane = threadIdx.x & 63;
  // uniform in the wavefront; saying so keeps the values derived from it (the
  // K-split index, the weight rows' base) in scalar registers, so the weight
  // loads take their K offset as a scalar operand
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);

  // ---- which (expert, row tile, piece of it, column tile) this workgroup computes
  // (with a second pass merged in, an expert's tiles are its first-pass tiles
  // followed by its overflow tiles, and its tile offset is the sum of both)
  const bool two = p.tile_off2 != nullptr;
  auto tiles_before = [&](int i) { return p.tile_off[i] + (two ? p.tile_off2[i] : 0); };
  const int NT = (p.N + G::BN - 1) / G::BN;
  const int ntiles = p.n_tiles[0] + (two ? p.n_tiles2[0] : 0);
  const int total = ntiles * NT * RS * KS;
  const int j = blockIdx.x >> 3;
  // Skew test, identical in every workgroup: are some experts' tile counts
  // well above the mean over active experts (max * active > 2 * tiles)?
  bool skewed = false;
  if (p.skew_map) {
    int mx = 0, act = 0;
    for (int b = 0; b < p.E; b += 64) {
      const int i = b + lane;
      const int t = (i < p.E) ? tiles_before(i + 1) - tiles_before(i) : 0;
      mx = max(mx, t);
      act += __popcll(__ballot(t > 0));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = max(mx, __shfl_xor(mx, o));
    // uniform by construction; saying so keeps the tile entry and the values
    // derived from it in scalar registers
    mx = __builtin_amdgcn_readfirstlane(mx);
    skewed = (long long)mx * act > 2LL * ntiles;
  }
  int L;
  if (!skewed) {
    const int J = (total + 7) >> 3;
    if (j >= J) return;
    L = (blockIdx.x & 7) * J + j;
  } else {
    L = ((j / kXcdChunk) * 8 + (blockIdx.x & 7)) * kXcdChunk + j % kXcdChunk;
  }
  if (L >= total) return;
  // K split: the KS workgroups of a unit are consecutive in L
  const int ks = L % KS;
  L /= KS;
  // expert e owns units [tiles_before(e) * NT * RS, tiles_before(e+1) * NT * RS),
  // column tile major, then row tile, then piece
  int e = 0;
  for (int b = 0; b <= p.E; b += 64) {
    const int i = b + lane;
    bool le = false;
    if (i >= 1 && i <= p.E) le = (long long)tiles_before(i) * NT * RS <= (long long)L;
    e += __popcll(__ballot(le));
  }
  const int t0 = tiles_before(e);
  const int mt = tiles_before(e + 1) - t0;
  const int local = L - t0 * NT * RS;
  const int nt = local / (mt * RS);
  const int rem = local - nt * mt * RS;
  const int ti = rem / RS;                            // tile of the expert
  const int mt1 = p.tile_off[e + 1] - p.tile_off[e];  // of them in the first pass
  const int4 ent = ti < mt1 ? reinterpret_cast<const int4*>(p.tile_map)[p.tile_off[e] + ti]
                            : reinterpret_cast<const int4*>(p.tile_map2)[p.tile_off2[e] + ti - mt1];
  const int piece = rem % RS;
  const int row0 = ent.y + piece * BM;           // first row of this workgroup
  const int rows = min(BM, ent.z - piece * BM);  // rows of this piece
  if (rows <= 0) return;

  typename G::Ctx c;
  {
    char* const all[8] = {st0, st1, st2, st3, st4, st5, st6, st7};
    setup_ctx<G>(c, p, all, e, row0, rows, nt * G::BN, wave, lane);
  }
  if constexpr (KS == 2) {
    const int nk = c.nk;  // steps of the whole K loop: the first range takes the larger half
    const int half = (nk + 1) / 2;
    c.s0 = ks == 0 ? 0 : half;
    c.nk = ks == 0 ? half : nk - half;
    c.nit = c.nk;
    // fp32 partial sums of range ks: plane ks of the [2][R][N] buffer
    c.ldo = (size_t)p.N * sizeof(float);
    c.out = reinterpret_cast<char*>(p.kpart + (size_t)ks * p.kplane) + (size_t)row0 * c.ldo;
  }
  // the weights are read by this workgroup alone if the expert's rows all fit in it
  G::template run_ms<G::MSUB>((rows + 15) >> 4, mt == 1 && ent.z <= BM, c);
}

// Fused gate+up over one pass of a tile map, with two column widths in one
// launch.  CN is the configuration of the map's tile height (WTN weight rows
// per wavefront); CW covers twice the columns per workgroup with the same
// wavefronts (twice the weight rows each), so every activation tile loaded
// into LDS feeds twice the weight bytes, but its accumulators fit in the
// registers only for tiles of at most CW::BM rows.  Each tile of at most
// CW::BM rows (in a map of CN::BM-row tiles only an expert's last tile can be
// one) is worked in units of CW's width; the other tiles (more than CW::BM
// rows) in units of CN's width.  Units are ordered expert-major, then by
// column group of CW's width, so the units that read one slice of an
// expert's weights stay consecutive: in column group g, the expert's
// CW-width unit (if its last tile is short) and then its full tiles at the
// CN-width columns 2g and 2g + 1.
template <class Tr, class CW, class CN>
__global__ __launch_bounds__(64 * CN::WN) void grouped_gemm_wide_kernel(GemmArgs p) {
  using GW = Gemm<Tr, CW::BM, CW::WTN, CW::WN, 1, true, CW::PF, CW::NTMS, false, CW::WS>;
  using GN = Gemm<Tr, CN::BM, CN::WTN, CN::WN, 1, true, CN::PF, CN::NTMS, false, CN::WS>;
  static_assert(CW::WN == CN::WN && CW::WK == 1 && CN::WK == 1 && CW::RS == 1 && CN::RS == 1, "wide pair");
  static_assert(CW::BM < CN::BM && CN::BM <= 2 * CW::BM && GW::BN == 2 * GN::BN, "wide pair");
  constexpr int STAGE = GW::STAGE > GN::STAGE ? GW::STAGE : GN::STAGE;
  constexpr int NA = GW::NA > GN::NA ? GW::NA : GN::NA;
  __shared__ __attribute__((aligned(16))) char st0[STAGE];
  __shared__ __attribute__((aligned(16))) char st1[STAGE];
  __shared__ __attribute__((aligned(16))) char st2[STAGE];
  __shared__ __attribute__((aligned(16))) char st3[NA > 3 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st4[NA > 4 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st5[NA > 5 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st6[NA > 6 ? STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st7[NA > 7 ? STAGE : 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int NTw = (p.N + GW::BN - 1) / GW::BN;
  const int NTn = (p.N + GN::BN - 1) / GN::BN;
  const int4* map = reinterpret_cast<const int4*>(p.tile_map);
  // units of expert i: its last tile in CW's width if it has at most CW::BM rows
  auto units_of = [&](int i) {
    const int t0 = p.tile_off[i], t1 = p.tile_off[i + 1];
    if (t1 == t0) return 0;
    const int sm = map[t1 - 1].z <= CW::BM ? 1 : 0;
    return sm * NTw + (t1 - t0 - sm) * NTn;
  };
  // total units over the experts, 64 at a time
  int total = 0;
  for (int b = 0; b < p.E; b += 64) {
    const int i = b + lane;
    int su = i < p.E ? units_of(i) : 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) su += __shfl_xor(su, o);
    total += su;
  }
  total = __builtin_amdgcn_readfirstlane(total);
  // Units are always dealt to the XCDs in chunks of kXcdChunk consecutive
  // units (with skew_map set): an expert with a tile of more than CW::BM rows
  // has twice the units of the others, and contiguous per-XCD ranges would
  // put them on one or two XCDs.  Measured at the Mixtral shape, T = 512,
  // seeds 0 / 1 / 2 (seed 1 has one 149-row expert): gate+up 333 / 379 / 335
  // against 335 / 407 / 344 us with contiguous ranges.
  const bool chunked = p.skew_map != 0;
  const int j = blockIdx.x >> 3;
  int L;
  if (!chunked) {
    const int J = (total + 7) >> 3;
    if (j >= J) return;
    L = (blockIdx.x & 7) * J + j;
  } else {
    L = ((j / kXcdChunk) * 8 + (blockIdx.x & 7)) * kXcdChunk + j % kXcdChunk;
  }
  if (L >= total) return;
  // expert of unit L: the number of experts whose units all lie at or before L;
  // `before`: the units of the experts ahead of it
  int e = 0, before = 0, carry = 0;
  for (int b = 0; b < p.E; b += 64) {
    const int i = b + lane;
    const int u = i < p.E ? units_of(i) : 0;
    int inc = u;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int n = __shfl_up(inc, o);
      if (lane >= o) inc += n;
    }
    const bool done = i < p.E && carry + inc <= L;
    e += __popcll(__ballot(done));
    int bu = done ? u : 0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) bu += __shfl_xor(bu, o);
    before += bu;
    carry += __shfl(inc, 63);
  }
  e = __builtin_amdgcn_readfirstlane(e);
  before = __builtin_amdgcn_readfirstlane(before);
  const int t0 = p.tile_off[e];
  const int mt = p.tile_off[e + 1] - t0;
  const int sm = map[t0 + mt - 1].z <= CW::BM ? 1 : 0;  // short last tile
  const int big = mt - sm;
  const int local = L - before;
  const int cw = local / (sm + 2 * big);                 // column group
  const int slot = local - cw * (sm + 2 * big);
  char* const stages[8] = {st0, st1, st2, st3, st4, st5, st6, st7};
  if (slot < sm) {
    const int4 ent = map[t0 + mt - 1];
    typename GW::Ctx c;
    setup_ctx<GW>(c, p, stages, e, ent.y, ent.z, cw * GW::BN, wave, lane);
    GW::template run_ms<GW::MSUB>((ent.z + 15) >> 4, mt == 1, c);
  } else {
    const int s2 = slot - sm;
    const int cn = 2 * cw + s2 / big;  // CN-width column
    const int4 ent = map[t0 + s2 % big];
    typename GN::Ctx c;
    setup_ctx<GN>(c, p, stages, e, ent.y, ent.z, cn * GN::BN, wave, lane);
    // a tile of more than CW::BM rows has all of CN's subtiles (the constant
    // count leaves only that main loop after inlining)
    GN::template run_ms<GN::MSUB>(GN::MSUB, mt == 1, c);
  }
}

template <class Tr, class Pair>
hipError_t launch_wide(const GemmArgs& a, hipStream_t stream) {
  using CN = typename Pair::narrow;
  constexpr int BNn = CN::WN * CN::WTN;
  const int NTn = (a.N + BNn - 1) / BNn;
  const long long units = (long long)a.max_tiles * NTn;  // every tile in CN's width at most
  const long long round = a.skew_map ? 8LL * kXcdChunk : 8;
  const long long grid = ((units + round - 1) / round) * round;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_wide_kernel<Tr, typename Pair::wide, CN>), dim3((unsigned)grid),
                     dim3(64 * CN::WN), 0, stream, a);
  return hipGetLastError();
}

template <class Tr, class Cfg, bool GATED, bool WQ, int KS = 1>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t stream) {
  constexpr int BN = Cfg::WN * Cfg::WTN;
  const int NT = (a.N + BN - 1) / BN;
  const long long units = (long long)a.max_tiles * NT * Cfg::RS * KS;
  const long long round = a.skew_map ? 8LL * kXcdChunk : 8;  // chunked mapping: whole rounds of chunks
  const long long grid = ((units + round - 1) / round) * round;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_kernel<Tr, Cfg::BM, Cfg::WTN, Cfg::WN, Cfg::WK, GATED, Cfg::PF, Cfg::NTMS, WQ, Cfg::RS,
                                         Cfg::WS, KS, Cfg::PP>),
                     dim3((unsigned)grid), dim3(64 * Cfg::WN * Cfg::WK), 0, stream, a);
  return hipGetLastError();
}

// Down GEMM of a decode batch with the combine folded in (16-row tile map,
// one pass).  Workgroup b owns output columns [b BN, b BN + BN) of every
// tile: it runs the down GEMM's main loop for each tile of the map in turn
// (the same Gemm, so y is bitwise that of grouped_gemm_kernel), stores y,
// and once every tile is done weights the rows of each token into its output
// for those columns exactly as the separate combine does (fp32 fmaf in slot
// order from 0, one rounding).  It saves the combine's launch; each
// workgroup streams the weights of every active expert for its columns.
template <class Tr, class Cfg, bool WQ>
__global__ __launch_bounds__(64 * Cfg::WN * Cfg::WK) void down_combine_kernel(GemmArgs p) {
  using G = Gemm<Tr, Cfg::BM, Cfg::WTN, Cfg::WN, Cfg::WK, false, Cfg::PF, Cfg::NTMS, WQ, Cfg::WS>;
  using Elt = typename Tr::T;
  constexpr int EPC = Tr::EPC;
  static_assert(Cfg::RS == 1 && Cfg::PP == 0 && G::BN % EPC == 0, "decode down + combine shape");
  __shared__ __attribute__((aligned(16))) char st0[G::STAGE];
  __shared__ __attribute__((aligned(16))) char st1[G::STAGE];
  __shared__ __attribute__((aligned(16))) char st2[G::STAGE];
  __shared__ __attribute__((aligned(16))) char st3[G::NA > 3 ? G::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st4[G::NA > 4 ? G::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st5[G::NA > 5 ? G::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st6[G::NA > 6 ? G::STAGE : 16];
  __shared__ __attribute__((aligned(16))) char st7[G::NA > 7 ? G::STAGE : 16];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nbase = (int)blockIdx.x * G::BN;
  if (nbase >= p.N) return;
  char* const all[8] = {st0, st1, st2, st3, st4, st5, st6, st7};
  const int ntiles = p.n_tiles[0];
  const int4* map = reinterpret_cast<const int4*>(p.tile_map);
  for (int i = 0; i < ntiles; ++i) {
    const int4 ent = map[i];
    const int mt = p.tile_off[ent.x + 1] - p.tile_off[ent.x];
    typename G::Ctx c;
    setup_ctx<G>(c, p, all, ent.x, ent.y, ent.z, nbase, wave, lane);
    G::template run_ms<G::MSUB>((ent.z + 15) >> 4, mt == 1 && ent.z <= Cfg::BM, c);
    // the next tile reuses the LDS stages; the last one's y rows are read below
    __syncthreads();
  }
  // combine of this workgroup's columns
  const size_t row_bytes = (size_t)p.N * sizeof(Elt);
  const int nch = min(G::BN, p.N - nbase) / EPC;  // 16-byte chunks of the slice
  const char* y = reinterpret_cast<const char*>(p.out);
  char* out = reinterpret_cast<char*>(p.comb_out);
  for (int idx = threadIdx.x; idx < p.comb_T * nch; idx += blockDim.x) {
    const int t = idx / nch;
    const size_t off = (size_t)(nbase + (idx - t * nch) * EPC) * sizeof(Elt);
    float acc[EPC];
#pragma unroll
    for (int q = 0; q < EPC; ++q) acc[q] = 0.f;
    for (int j = 0; j < p.comb_k; ++j) {
      const int row = p.comb_row_of[(size_t)t * p.comb_k + j];
      if (row < 0) continue;
      const float wj = p.comb_w[(size_t)t * p.comb_k + j];
      float v[EPC];
      widen<Tr>(*reinterpret_cast<const uint4*>(y + (size_t)row * row_bytes + off), v);
#pragma unroll
      for (int q = 0; q < EPC; ++q) acc[q] = fmaf(wj, v[q], acc[q]);
    }
    *reinterpret_cast<uint4*>(out + (size_t)t * row_bytes + off) = narrow<Tr>(acc);
  }
}

template <class Tr, bool WQ>
hipError_t launch_down_combine(const GemmArgs& a, hipStream_t stream) {
  using Cfg = typename TileCfg<16, false, WQ>::type;
  constexpr int BN = Cfg::WN * Cfg::WTN;
  const int grid = (a.N + BN - 1) / BN;
  hipLaunchKernelGGL((down_combine_kernel<Tr, Cfg, WQ>), dim3((unsigned)grid), dim3(64 * Cfg::WN * Cfg::WK), 0,
                     stream, a);
  return hipGetLastError();
}

template <class Tr, bool GATED, bool WQ = false>
hipError_t dispatch_bm(int BM, const GemmArgs& a, hipStream_t stream) {
  if constexpr (GATED && !WQ && std::is_same<Tr, TBF16>::value) {
    if (BM == 160 && a.wide && a.tile_off2 == nullptr) return launch_wide<Tr, Wide160>(a, stream);
  }
  if constexpr (!GATED && std::is_same<Tr, TBF16>::value) {
    if (BM == 160 && a.kpart != nullptr) return launch_cfg<Tr, Split160, false, WQ, 2>(a, stream);
  }
  if constexpr (!GATED) {
    if (a.comb_out != nullptr) return BM == 16 ? launch_down_combine<Tr, WQ>(a, stream) : hipErrorInvalidValue;
  }
  switch (BM) {
#define MOE_BM_CASE(bm) \
  case bm:              \
    return launch_cfg<Tr, typename TileCfg<bm, GATED, WQ>::type, GATED, WQ>(a, stream);
    MOE_BM_CASE(16)
    MOE_BM_CASE(32)
    MOE_BM_CASE(48)
    MOE_BM_CASE(64)
    MOE_BM_CASE(96)
    MOE_BM_CASE(128)
    MOE_BM_CASE(160)
    MOE_BM_CASE(192)
    MOE_BM_CASE(384)
#undef MOE_BM_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gemm
}  // namespace moe
