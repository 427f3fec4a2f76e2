// Block-scheduled grouped GEMMs of the expert FFN on the gfx950 matrix cores.
//
// TritonMoE review (pith.science verdict for arXiv 2605.23911): the expert
// GEMMs run as one grouped GEMM whose fixed-size program blocks are mapped
// to (expert, token offset) pairs (referee summary, Algorithm 1, section
// 3.2); the gate and up projections share each load of the input tile and
// SiLU(gate) * up is formed in registers, so neither projection is written
// to memory (key machinery); the down projection is a separate kernel
// (desk-editor letter).
//
// Both GEMMs are "NT": activations [rows][K] and weights [N][K] are K-contiguous.
// A workgroup owns one (row tile, column tile) pair.  Which pair comes from
// the tile map that the dispatch step wrote on the device: the tile count is
// read on the device and excess workgroups of the static grid exit at once.
//
// Data movement, per 128-byte K step:
//  - the activation tile (BM rows) is loaded by the whole workgroup into a
//    double-buffered LDS tile (rows padded to 144 bytes so 16-byte lane reads
//    of 16 consecutive rows hit distinct banks) and read by every wavefront;
//  - weights are streamed by each wavefront straight into MFMA operand
//    registers, PF K-steps ahead, with no LDS round trip: a wavefront owns
//    WTN weight rows (per projection), so no weight byte is shared between
//    wavefronts, and every weight byte is read from HBM once per row tile.
// Weights are the MFMA "A" operand (output rows = weight rows n) and the
// activations the "B" operand (output columns = token rows m), so each lane
// ends with 4 consecutive n of one row m, stored as one 8- or 16-byte write.
//
// Workgroup order is XCD-aware: gfx950 hands consecutive workgroup ids to its
// 8 XCDs round-robin, so id b is remapped to linear unit (b mod 8) * J + b / 8
// (J = units per XCD).  Each XCD therefore walks a contiguous range of units,
// ordered expert-major, then column tile, then row tile: the row tiles that
// share one weight column tile run back to back on one XCD and share its L2,
// and the activation rows of one expert stay in that XCD's L2.
#include <limits.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kKB = 128;               // bytes of K per pipeline step
constexpr int kLdsStride = kKB + 16;   // padded LDS row stride (bytes)

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

template <class Tr, int BM, int WTN, int WN, bool GATED, int PF>
__global__ __launch_bounds__(64 * WN) void grouped_gemm_kernel(GemmArgs p) {
  using Elt = typename Tr::T;
  constexpr int NTH = 64 * WN;
  constexpr int NSUB = WTN / 16;
  constexpr int NMAT = GATED ? 2 : 1;
  constexpr int MSUB = BM / 16;
  constexpr int WL = NMAT * NSUB * 2;           // 16-byte weight loads per lane per step
  constexpr int ACH = BM * (kKB / 16);          // 16-byte chunks of the activation tile
  constexpr int APT = (ACH + NTH - 1) / NTH;    // chunks per thread
  constexpr int BN = WN * WTN;                  // output columns per workgroup
  static_assert(WTN % 16 == 0 && BM % 16 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) char lds[2][BM * kLdsStride];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  // ---- which (expert, row tile, column tile) this workgroup computes
  const int NT = p.N / BN;
  const int total = p.n_tiles[0] * NT;
  const int J = (total + 7) >> 3;
  const int j = blockIdx.x >> 3;
  if (j >= J) return;
  const int L = (blockIdx.x & 7) * J + j;
  if (L >= total) return;
  // expert e owns units [tile_off[e] * NT, tile_off[e+1] * NT)
  int e = 0;
  for (int b = 0; b <= p.E; b += 64) {
    const int i = b + lane;
    bool le = false;
    if (i >= 1 && i <= p.E) le = (long long)p.tile_off[i] * NT <= (long long)L;
    e += __popcll(__ballot(le));
  }
  const int t0 = p.tile_off[e];
  const int mt = p.tile_off[e + 1] - t0;
  const int local = L - t0 * NT;
  const int nt = local / mt;
  const int4 ent = reinterpret_cast<const int4*>(p.tile_map)[t0 + (local - nt * mt)];
  const int row0 = ent.y;
  const int rows = ent.z;
  const int n0 = nt * BN + wave * WTN;

  const size_t ld = (size_t)p.K * sizeof(Elt);  // bytes per row (activations and weights)
  const char* act = reinterpret_cast<const char*>(p.act) + (size_t)row0 * ld;
  const size_t wexp = (size_t)p.N * ld;
  const char* wsrc[NMAT];
  wsrc[0] = reinterpret_cast<const char*>(p.w0) + (size_t)e * wexp + (size_t)n0 * ld;
  if (GATED) wsrc[NMAT - 1] = reinterpret_cast<const char*>(p.w1) + (size_t)e * wexp + (size_t)n0 * ld;
  const size_t wlane = (size_t)(lane & 15) * ld + (lane >> 4) * 16;

  const int nsteps = (int)(ld / kKB);

  f32x4_t acc[NMAT][NSUB][MSUB];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < NSUB; ++i)
#pragma unroll
      for (int jm = 0; jm < MSUB; ++jm) acc[m][i][jm] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  uint4 wq[PF][WL];
  uint4 areg[APT];

  auto load_w = [&](int s, uint4* dst) {
    const size_t ko = (size_t)s * kKB + wlane;
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int i = 0; i < NSUB; ++i)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          dst[(m * NSUB + i) * 2 + h] =
              *reinterpret_cast<const uint4*>(wsrc[m] + (size_t)i * 16 * ld + ko + h * 64);
  };
  auto load_a = [&](int s) {
#pragma unroll
    for (int q = 0; q < APT; ++q) {
      const int c = threadIdx.x + q * NTH;
      const int r = c >> 3;
      uint4 v = make_uint4(0, 0, 0, 0);
      if ((ACH % NTH == 0 || c < ACH) && r < rows)
        v = *reinterpret_cast<const uint4*>(act + (size_t)r * ld + (size_t)s * kKB + (c & 7) * 16);
      areg[q] = v;
    }
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int q = 0; q < APT; ++q) {
      const int c = threadIdx.x + q * NTH;
      if (ACH % NTH == 0 || c < ACH)
        *reinterpret_cast<uint4*>(&lds[buf][(c >> 3) * kLdsStride + (c & 7) * 16]) = areg[q];
    }
  };

  // prologue
#pragma unroll
  for (int u = 0; u < PF; ++u)
    if (u < nsteps) load_w(u, wq[u]);
  load_a(0);
  store_a(0);
  __syncthreads();

  for (int s0 = 0; s0 < nsteps; s0 += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) {
      const int s = s0 + u;
      if (s < nsteps) {
        const bool more = s + 1 < nsteps;
        if (more) load_a(s + 1);
        const char* lb = lds[s & 1];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uint4 af[MSUB];
#pragma unroll
          for (int jm = 0; jm < MSUB; ++jm)
            af[jm] = *reinterpret_cast<const uint4*>(lb + (jm * 16 + (lane & 15)) * kLdsStride + h * 64 +
                                                     (lane >> 4) * 16);
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int i = 0; i < NSUB; ++i)
#pragma unroll
              for (int jm = 0; jm < MSUB; ++jm)
                acc[m][i][jm] = mma16<Tr>(wq[u][(m * NSUB + i) * 2 + h], af[jm], acc[m][i][jm]);
        }
        if (s + PF < nsteps) load_w(s + PF, wq[u]);
        if (more) store_a((s + 1) & 1);
        __syncthreads();
      }
    }
  }

  // ---- epilogue: lane holds rows n = n0 + 16 i + 4 (lane/16) + r of column m
  char* out = reinterpret_cast<char*>(p.out);
  const size_t ldo = (size_t)p.N * sizeof(Elt);
#pragma unroll
  for (int jm = 0; jm < MSUB; ++jm) {
    const int m = jm * 16 + (lane & 15);
    if (m < rows) {
      char* orow = out + (size_t)(row0 + m) * ldo;
#pragma unroll
      for (int i = 0; i < NSUB; ++i) {
        const int n = n0 + i * 16 + (lane >> 4) * 4;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
          v[r] = GATED ? silu_mul(acc[0][i][jm][r], acc[NMAT - 1][i][jm][r]) : acc[0][i][jm][r];
        store4<Tr>(orow + (size_t)n * sizeof(Elt), v[0], v[1], v[2], v[3]);
      }
    }
  }
}

template <class Tr, int BM, int WTN, int WN, bool GATED, int PF>
hipError_t launch_one(const GemmArgs& a, hipStream_t stream) {
  constexpr int BN = WN * WTN;
  const int NT = a.N / BN;
  const long long units = (long long)a.max_tiles * NT;
  const long long grid = ((units + 7) / 8) * 8;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((grouped_gemm_kernel<Tr, BM, WTN, WN, GATED, PF>), dim3((unsigned)grid), dim3(64 * WN), 0,
                     stream, a);
  return hipGetLastError();
}

template <class Tr, bool GATED>
hipError_t dispatch_bm(int BM, const GemmArgs& a, hipStream_t stream) {
  switch (BM) {
    case 16: return launch_one<Tr, 16, 16, 4, GATED, GATED ? 4 : 8>(a, stream);
    case 32: return launch_one<Tr, 32, 16, 4, GATED, GATED ? 4 : 8>(a, stream);
    case 64: return launch_one<Tr, 64, 16, 4, GATED, GATED ? 4 : 8>(a, stream);
    case 128: return launch_one<Tr, 128, 16, 4, GATED, GATED ? 4 : 6>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

GemmTiling gemm_tiling(int BM, bool gated, int N) {
  (void)gated;
  (void)N;
  return GemmTiling{BM, 64, 256};
}

hipError_t launch_grouped_gemm(int dtype, bool gated, int BM, const GemmArgs& a, hipStream_t stream) {
  if (dtype == 1) return gated ? dispatch_bm<TBF16, true>(BM, a, stream) : dispatch_bm<TBF16, false>(BM, a, stream);
  return gated ? dispatch_bm<TF32, true>(BM, a, stream) : dispatch_bm<TF32, false>(BM, a, stream);
}

}  // namespace moe
