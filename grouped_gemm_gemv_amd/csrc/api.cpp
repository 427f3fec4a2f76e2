// C ABI of libmoe: host-side validation, sizing, workspace layout and kernel
// enqueue.  Nothing here allocates, frees or synchronises; every validation
// error is returned before the first HIP call.
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "launch.hpp"
#include "moe.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Largest row-tile height of the grouped GEMMs.  A tile holds up to BM rows
// and only its non-empty 16-row subtiles are computed, so a tall tile costs
// nothing for short experts.  The configurations come in two families:
//  * tall (BM 160/192/384: 112- to 256-column workgroups, K not split) stream
//    weights best and give a hot expert the fewest row tiles, but need many
//    column tiles to occupy the 256 compute units;
//  * short (BM 16/32: 32 columns, K split over 4 wavefronts; BM 48/64: 64
//    columns, K split over 2) multiply the workgroups without duplicating a
//    weight stream, for few active experts.
// The rule below was fitted to per-expert cost curves measured on this GPU
// (Mixtral, 64-expert and capacity shapes, blocked weights); each branch
// states the measurement behind it.  The mean is T*k over min(E, T*k)
// experts, at most C in the capacity pass.
constexpr int kTileRows[] = {16, 32, 48, 64, 96, 128, 160, 192, 384};
constexpr int kComputeUnits = 256;

bool supported_tile_rows(int bm) {
  for (int v : kTileRows)
    if (v == bm) return true;
  return false;
}

int choose_tile_rows(const moe_shape_t& s) {
  if (s.tile_rows != 0) return s.tile_rows;
  const int64_t Tk = (int64_t)s.T * s.k;
  const int64_t active = std::min<int64_t>(s.E, Tk);
  int64_t mean = ceil_div(Tk, active);
  if (s.capacity > 0) mean = std::min<int64_t>(mean, s.capacity);
  // A token or two per expert: 16-row split-K tiles stream the weights best.
  if (mean <= 2) return 16;
  // Tall tiles once enough of them exist to fill the units; a lone expert stays
  // on 64-row split-K tiles up to 512 rows (one Mixtral expert: 64 rows 143 us,
  // 160 rows 197 us at 256 rows).
  const int64_t tall_tiles = active * ceil_div(s.d, 128);
  if (tall_tiles >= kComputeUnits * 3 / 4 || (mean > 64 && tall_tiles >= 64) || mean > 512) {
    // 192 rows (256-column down tiles) once there are many such tiles; past 160
    // rows also with fewer, unless 160-row tiles pad less below 320 rows.  On
    // 8 experts of d = 3584: 64 rows 85 us at 160 vs 91 at 192, 192 rows 193 vs
    // 155 us; 8 Mixtral experts of 192 rows: 1001 vs 748 us; 32 or more
    // experts of d = 3584: 192 ahead by 2-7 %.
    // 193-256 rows: two balanced 128-row tiles.  Measured per-expert cost
    // curves, 224 / 256 rows: 8 Mixtral experts 775 / 813 us at 128 against
    // 870 / 882 at 160 and 929 / 918 at 192; 32 experts of d = 2048,
    // F = 1408: 173 / 181 us against 216 / 212 at 192.
    if (mean > 192 && mean <= 256) return 128;
    const int64_t r192 = ceil_div(mean, 192);
    const int64_t w192 = active * r192 * ceil_div(s.d, 256);
    const bool past160 = w192 >= 112 && mean > 160 &&
                         (mean > 320 || r192 * 192 <= ceil_div(mean, 160) * 160);
    if (!(w192 >= 448 || past160)) return 160;
    // A thousand rows or more per expert, or past 384 rows with large experts
    // (d * F of 2^25 or more): 384-row tiles, which gate+up works in 128-row
    // pieces with 32 weight rows per wavefront (twice the MFMAs per
    // activation fragment read from LDS) and down in 192-row pieces, both
    // with the ping-pong main loop.  Per-expert cost curves with these
    // kernels: 8 Mixtral experts (d * F = 58.7M) of 448 / 512 / 640 / 768
    // rows 1268 / 1321 / 1696 / 1817 us against 1406 / 1461 / 1733 / 1864 at
    // 192, of 384 rows 1024 against 1012; 32 experts of d = 2048, F = 1408
    // ahead at 192 up to 768 rows (448 rows: 303 vs 313 us) and behind at
    // 1024 (629 vs 580 us); 32 experts of d = 3584, F = 2560 within 2 % at
    // 448-768 rows.  Experts shorter than a tile leave pieces empty, whose
    // workgroups still hold a compute unit while they find that out.
    const bool large = (int64_t)s.d * s.F >= (int64_t(1) << 25);
    return (mean >= 1024 || (large && mean > 384)) ? 384 : 192;
  }
  if (mean > 32) return 64;
  if (active * ceil_div(s.d, 64) >= kComputeUnits) return 48;
  return (mean * 5 + 3) / 4 <= 16 ? 16 : 32;
}

int64_t mean_rows(const moe_shape_t& s) {
  const int64_t Tk = (int64_t)s.T * s.k;
  int64_t mean = ceil_div(Tk, std::min<int64_t>(s.E, Tk));
  if (s.capacity > 0) mean = std::min<int64_t>(mean, s.capacity);
  return mean;
}

// The bf16 down GEMM on the 160-row tile map splits its K loop in two
// (Split160 in gemm_tiles.hpp) from this many mean rows per expert, where the
// activation bytes moved into LDS weigh about as much as the weight bytes.
// Measured, 8 Mixtral experts, down GEMM with the kernel adding the two
// halves: 64 rows 152 vs 143 us, 96 rows 155 vs 162, 128 rows 164 vs 179,
// 144 rows 168 vs 191.
constexpr int kSplitMinRows = 80;

bool split_down(const moe_shape_t& s, int BM) {
  return BM == 160 && s.dtype == MOE_BF16 && mean_rows(s) >= kSplitMinRows && (int64_t)s.F * 2 >= 256;
}

// moe_forward folds the combine into the down GEMM for a batch of at most
// two (token, slot) entries on the 16-row tile map, one pass: each down
// workgroup computes its column slice of y for every tile and then the output
// columns of every token (down_combine_kernel), which saves the combine's
// launch.  Each workgroup then streams every active expert's weights for its
// columns, so there are as many workgroups as column tiles instead of tiles
// times column tiles.  Measured at the Mixtral shape: T = 1 (two tiles) 125.0
// vs 126.2 us per layer; T = 8 (up to eight tiles) 386.1 vs 383.5, hence the
// limit.  With 8 wavefronts splitting K instead of 4 the gain at T = 1 was
// gone (126.3 us).
bool fused_down_combine(const moe_shape_t& s, int BM) {
  return BM == 16 && s.capacity == 0 && (int64_t)s.T * s.k <= 2;
}

int64_t spill_bound(const moe_shape_t& s) { return std::max<int64_t>(0, (int64_t)s.T * s.k - s.capacity); }

// Upper bound on the tiles of one pass: a pass of R_p rows over at most E_p
// non-empty experts has sum ceil(r_e / BM) <= (R_p + E_p (BM - 1)) / BM.
int64_t pass_max_tiles(const moe_shape_t& s, int BM, int pass) {
  const int64_t Tk = (int64_t)s.T * s.k;
  if (s.capacity <= 0) {
    if (pass == 1) return 0;
    return (Tk + std::min<int64_t>(s.E, Tk) * (BM - 1)) / BM;
  }
  const int64_t C = s.capacity;
  if (pass == 0) {
    const int64_t Rp = std::min<int64_t>(Tk, (int64_t)s.E * C);
    return std::min<int64_t>((Rp + std::min<int64_t>(s.E, Tk) * (BM - 1)) / BM, (int64_t)s.E * ceil_div(C, BM));
  }
  const int64_t Ep = std::min<int64_t>(s.E, Tk / (C + 1));  // overflowing experts hold >= C+1 entries
  return (spill_bound(s) + Ep * (BM - 1)) / BM;
}

int64_t row_space(const moe_shape_t& s) {
  if (s.capacity <= 0) return (int64_t)s.T * s.k;
  return (int64_t)s.E * s.capacity + spill_bound(s);
}

size_t elt_bytes(const moe_shape_t& s) { return s.dtype == MOE_BF16 ? 2 : 4; }

// The GEMM kernels address their operands with 32-bit buffer offsets:
//  * a workgroup's weight descriptor spans up to 256 rows, and its lanes'
//    offsets up to 256 rows plus the K loop, so one weight or activation row
//    (d or F elements) may take at most kMaxRowBytes;
//  * with the gather folded into the gate+up loads, a lane's offset into x is
//    token * row bytes + the K position, and padding rows of a tile read at
//    kPadOffset (past the end of x, so they return zeros), plus the K
//    position: x may take at most kPadOffset bytes.
constexpr int64_t kMaxRowBytes = int64_t(1) << 20;
constexpr int64_t kPadOffset = 0x7ff00000;

moe_status_t validate(const moe_shape_t* s) {
  if (s == nullptr) return MOE_ERR_NULL_PTR;
  if (s->T < 1 || s->E < 1 || s->E > 256 || s->k < 1 || s->k > s->E || s->k > 64 || s->capacity < 0 ||
      s->d < 64 || s->F < 64)
    return MOE_ERR_INVALID_ARG;
  if (s->dtype != MOE_F32 && s->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (s->tile_rows != 0 && !supported_tile_rows(s->tile_rows)) return MOE_ERR_UNSUPPORTED;
  if (s->weight_layout != MOE_LAYOUT_ROWS && s->weight_layout != MOE_LAYOUT_BLOCKED16) return MOE_ERR_INVALID_ARG;
  if (s->d % 64 != 0 || s->F % 64 != 0) return MOE_ERR_UNSUPPORTED;
  const int64_t eb = s->dtype == MOE_BF16 ? 2 : 4;
  if ((int64_t)s->d * eb > kMaxRowBytes || (int64_t)s->F * eb > kMaxRowBytes) return MOE_ERR_UNSUPPORTED;
  const int64_t Tk = (int64_t)s->T * s->k;
  if (Tk >= INT32_MAX) return MOE_ERR_INVALID_ARG;
  const int64_t R = row_space(*s);
  if (R >= INT32_MAX) return MOE_ERR_INVALID_ARG;
  if ((int64_t)s->E * s->capacity >= INT32_MAX) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// The gate+up GEMM reads x through token_of (see kPadOffset).
moe_status_t validate_gather(const moe_shape_t& s) {
  const int64_t eb = s.dtype == MOE_BF16 ? 2 : 4;
  return (int64_t)s.T * s.d * eb <= kPadOffset ? MOE_OK : MOE_ERR_UNSUPPORTED;
}

// Layout of the dispatch buffer (byte offsets from its base).
struct DispatchLayout {
  size_t counts, offsets, spill_counts, spill_offsets, row_of, token_of, tile_off, tile_map, n_tiles, err_flags;
  size_t kpart;
  size_t bytes;
};

struct Plan {
  int64_t Tk, R;
  int BM;
  bool ksplit;            // the bf16 down GEMM splits K in two (Split160): [2][R][d] fp32 partial sums
  int64_t max_tiles;      // stride of each pass in tile_map
  int64_t pass_tiles[2];  // grid bound of each pass
  int nblk;
  DispatchLayout dl;
  size_t permute_ws;      // block counts + block error flags
  size_t ws_ids, ws_w, ws_disp, ws_perm, ws_h, ws_y, forward_ws;
};

Plan make_plan(const moe_shape_t& s) {
  Plan p{};
  p.Tk = (int64_t)s.T * s.k;
  p.R = row_space(s);
  p.BM = choose_tile_rows(s);
  p.pass_tiles[0] = pass_max_tiles(s, p.BM, 0);
  p.pass_tiles[1] = pass_max_tiles(s, p.BM, 1);
  p.max_tiles = std::max<int64_t>(1, std::max(p.pass_tiles[0], p.pass_tiles[1]));
  p.ksplit = split_down(s, p.BM);
  p.nblk = (int)ceil_div(p.Tk, moe::kCountChunk);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  const size_t E = (size_t)s.E;
  p.dl.counts = take(4 * E);
  p.dl.offsets = take(4 * (E + 1));
  p.dl.spill_counts = take(4 * E);
  p.dl.spill_offsets = take(4 * (E + 1));
  p.dl.row_of = take(4 * (size_t)p.Tk);
  p.dl.token_of = take(4 * (size_t)p.R);
  p.dl.tile_off = take(4 * 2 * (E + 1));
  p.dl.tile_map = take(4 * 4 * 2 * (size_t)p.max_tiles);
  p.dl.n_tiles = take(4 * 2);
  p.dl.err_flags = take(4);
  p.dl.kpart = take(p.ksplit ? 4 * 2 * (size_t)p.R * s.d : 0);
  p.dl.bytes = o;
  p.permute_ws = align_up(4 * (size_t)p.nblk * E) + align_up(4 * (size_t)p.nblk);
  const size_t eb = elt_bytes(s);
  o = 0;
  p.ws_ids = take(4 * (size_t)p.Tk);
  p.ws_w = take(4 * (size_t)p.Tk);
  p.ws_disp = take(p.dl.bytes);
  p.ws_perm = take(p.permute_ws);
  p.ws_h = take((size_t)p.R * s.F * eb);
  p.ws_y = take((size_t)p.R * s.d * eb);
  p.forward_ws = o;
  return p;
}

void carve(const moe_shape_t& s, const Plan& p, char* base, moe_dispatch_t* d) {
  d->counts = reinterpret_cast<int32_t*>(base + p.dl.counts);
  d->offsets = reinterpret_cast<int32_t*>(base + p.dl.offsets);
  d->spill_counts = reinterpret_cast<int32_t*>(base + p.dl.spill_counts);
  d->spill_offsets = reinterpret_cast<int32_t*>(base + p.dl.spill_offsets);
  d->row_of = reinterpret_cast<int32_t*>(base + p.dl.row_of);
  d->token_of = reinterpret_cast<int32_t*>(base + p.dl.token_of);
  d->tile_off = reinterpret_cast<int32_t*>(base + p.dl.tile_off);
  d->tile_map = reinterpret_cast<int32_t*>(base + p.dl.tile_map);
  d->n_tiles = reinterpret_cast<int32_t*>(base + p.dl.n_tiles);
  d->err_flags = reinterpret_cast<uint32_t*>(base + p.dl.err_flags);
  d->kpart = p.ksplit ? reinterpret_cast<float*>(base + p.dl.kpart) : nullptr;
  d->tile_rows = p.BM;
  d->max_tiles = (int32_t)p.max_tiles;
  (void)s;
}

moe_status_t check_dispatch(const moe_shape_t& s, const Plan& p, const moe_dispatch_t* d) {
  if (d == nullptr) return MOE_ERR_NULL_PTR;
  if (!d->counts || !d->offsets || !d->spill_counts || !d->spill_offsets || !d->row_of || !d->token_of ||
      !d->tile_off || !d->tile_map || !d->n_tiles || !d->err_flags)
    return MOE_ERR_NULL_PTR;
  if (split_down(s, d->tile_rows) && d->kpart == nullptr) return MOE_ERR_NULL_PTR;
  if (!supported_tile_rows(d->tile_rows)) return MOE_ERR_UNSUPPORTED;
  const int64_t need = std::max(pass_max_tiles(s, d->tile_rows, 0), pass_max_tiles(s, d->tile_rows, 1));
  if (d->max_tiles < need || d->max_tiles < 1) return MOE_ERR_INVALID_ARG;
  (void)p;
  return MOE_OK;
}

moe_status_t hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe::SmallDispatchArgs small_dispatch_args(const moe_shape_t& s, const Plan& p, const int32_t* ids,
                                           const moe_dispatch_t& d) {
  moe::SmallDispatchArgs a;
  a.ids = ids;
  a.Tk = (int)p.Tk;
  a.k = s.k;
  a.E = s.E;
  a.C = s.capacity;
  a.BM = d.tile_rows;
  a.max_tiles = d.max_tiles;
  a.rows = p.R;
  a.counts = d.counts;
  a.offsets = d.offsets;
  a.spill_counts = d.spill_counts;
  a.spill_offsets = d.spill_offsets;
  a.row_of = d.row_of;
  a.token_of = d.token_of;
  a.tile_off = d.tile_off;
  a.tile_map = d.tile_map;
  a.n_tiles = d.n_tiles;
  a.err_flags = d.err_flags;
  return a;
}

// Dispatch (count, scan, ranks, tile map) and, if x_perm is not null, the gather.
moe_status_t enqueue_permute(const moe_shape_t& s, const Plan& p, const void* x, const int32_t* ids,
                             const moe_dispatch_t& d, void* x_perm, void* ws, hipStream_t st) {
  char* w = static_cast<char*>(ws);
  int32_t* block_counts = reinterpret_cast<int32_t*>(w);
  uint32_t* block_err = reinterpret_cast<uint32_t*>(w + align_up(4 * (size_t)p.nblk * s.E));
  const int Tk = (int)p.Tk;
  if (Tk <= moe::kSmallDispatch) {
    if (moe::launch_dispatch_small(small_dispatch_args(s, p, ids, d), st) != hipSuccess) return MOE_ERR_HIP;
    if (x_perm == nullptr) return MOE_OK;
    return hip_status(moe::launch_gather(x, d.row_of, Tk, s.k, (int64_t)s.d * elt_bytes(s), x_perm, st));
  }
  hipError_t e = moe::launch_count(ids, Tk, s.E, p.nblk, block_counts, block_err, d.token_of, p.R, st);
  if (e != hipSuccess) return MOE_ERR_HIP;
  moe::ScanArgs a;
  a.block_counts = block_counts;
  a.block_err = block_err;
  a.nblk = p.nblk;
  a.E = s.E;
  a.C = s.capacity;
  a.BM = d.tile_rows;
  a.max_tiles = d.max_tiles;
  a.counts = d.counts;
  a.offsets = d.offsets;
  a.spill_counts = d.spill_counts;
  a.spill_offsets = d.spill_offsets;
  a.tile_off = d.tile_off;
  a.tile_map = d.tile_map;
  a.n_tiles = d.n_tiles;
  a.err_flags = d.err_flags;
  if ((e = moe::launch_scan(a, st)) != hipSuccess) return MOE_ERR_HIP;
  if ((e = moe::launch_scatter(ids, Tk, s.k, s.E, s.capacity, p.nblk, block_counts, d.offsets, d.spill_offsets,
                               d.row_of, d.token_of, st)) != hipSuccess)
    return MOE_ERR_HIP;
  if (x_perm == nullptr) return MOE_OK;
  return hip_status(moe::launch_gather(x, d.row_of, Tk, s.k, (int64_t)s.d * elt_bytes(s), x_perm, st));
}

// pass 0 or 1; kBothPasses: both passes of the capacity mode in one launch
constexpr int kBothPasses = MOE_PASS_BOTH;

moe::GemmArgs gemm_args(const moe_shape_t& s, const moe_dispatch_t& d, int pass, bool gated) {
  moe::GemmArgs a{};
  a.act_rows = nullptr;
  a.act_nrows = 0;
  const bool both = pass == kBothPasses && s.capacity > 0;
  const int p0 = pass == kBothPasses ? 0 : pass;
  a.tile_off = d.tile_off + p0 * (s.E + 1);
  a.tile_map = d.tile_map + (size_t)p0 * d.max_tiles * 4;
  a.n_tiles = d.n_tiles + p0;
  a.tile_off2 = nullptr;
  a.tile_map2 = nullptr;
  a.n_tiles2 = nullptr;
  a.max_tiles = (int)pass_max_tiles(s, d.tile_rows, p0);
  if (both) {
    a.tile_off2 = d.tile_off + (s.E + 1);
    a.tile_map2 = d.tile_map + (size_t)d.max_tiles * 4;
    a.n_tiles2 = d.n_tiles + 1;
    a.max_tiles += (int)pass_max_tiles(s, d.tile_rows, 1);
  }
  a.E = s.E;
  a.K = gated ? s.d : s.F;
  a.N = gated ? s.F : s.d;
  a.skew_map = 1;
  a.blocked16 = s.weight_layout == MOE_LAYOUT_BLOCKED16 ? 1 : 0;
  a.wide = 0;
  a.kpart = nullptr;
  a.kplane = 0;
  return a;
}

// Mean rows per expert for which the bf16 gate+up on the 160-row tile map
// takes the two-width kernel (Wide160 in gemm_tiles.hpp).  Measured, 8
// Mixtral experts: 3 % faster at 64 rows, 10 % at 128, 13 % at 140-144,
// 2-3 % faster even when every expert holds 148-160 rows (all of them in
// 112-column units, dealt to the XCDs in chunks), 2 % slower at 32.
constexpr int kWideMinRows = 48;
constexpr int kWideMaxRows = 160;


// Gate+up over one pass.  With x_src set, activation row r is read from row
// token_of[r] of x_src (the gather folded into the GEMM's loads); otherwise
// from row r of x_perm.
moe_status_t enqueue_gate_up(const moe_shape_t& s, const void* x_perm, const void* wg, const void* wu,
                             const moe_dispatch_t& d, int pass, void* h, hipStream_t st,
                             const void* x_src = nullptr, const float* sg = nullptr, const float* su = nullptr) {
  moe::GemmArgs a = gemm_args(s, d, pass, true);
  a.s0 = sg;
  a.s1 = su;
  const int64_t mean = mean_rows(s);
  a.wide = (sg == nullptr && s.dtype == MOE_BF16 && mean >= kWideMinRows && mean <= kWideMaxRows) ? 1 : 0;
  a.act = x_src != nullptr ? x_src : x_perm;
  a.act_rows = x_src != nullptr ? d.token_of : nullptr;
  a.act_nrows = s.T;
  a.w0 = wg;
  a.w1 = wu;
  a.out = h;
  return hip_status(moe::launch_grouped_gemm(s.dtype, true, d.tile_rows, a, st));
}

// Down GEMM over one pass.  With the K loop split (split_down), the two fp32
// partial planes are added into y by k_split_finish unless `finish` is false
// (moe_forward then forms y inside its combine).
moe_status_t enqueue_down(const moe_shape_t& s, const void* h, const void* wd, const moe_dispatch_t& d, int pass,
                          void* y, hipStream_t st, const float* sd = nullptr, bool finish = true,
                          void* comb_out = nullptr, const float* comb_w = nullptr) {
  moe::GemmArgs a = gemm_args(s, d, pass, false);
  a.s0 = sd;
  if (comb_out != nullptr) {
    a.comb_out = comb_out;
    a.comb_w = comb_w;
    a.comb_row_of = d.row_of;
    a.comb_T = s.T;
    a.comb_k = s.k;
  }
  const bool split = split_down(s, d.tile_rows);
  if (split) {
    a.kpart = d.kpart;
    a.kplane = (size_t)row_space(s) * s.d;
  }
  a.act = h;
  a.w0 = wd;
  a.w1 = nullptr;
  a.out = y;
  moe_status_t st_ = hip_status(moe::launch_grouped_gemm(s.dtype, false, d.tile_rows, a, st));
  if (st_ != MOE_OK || !split || !finish) return st_;
  // y rows of the pass(es) just computed: the uncapped rows or the fixed
  // region (pass 0), the overflow region (pass 1)
  const int64_t fixed = s.capacity > 0 ? (int64_t)s.E * s.capacity : row_space(s);
  const int64_t r0 = pass == 1 ? fixed : 0;
  const int64_t r1 = (pass == 0 && s.capacity > 0) ? fixed : row_space(s);
  return hip_status(moe::launch_k_split_finish(s.dtype, d.kpart + (size_t)r0 * s.d, a.kplane, d.token_of + r0, r1 - r0,
                                                s.d, static_cast<char*>(y) + (size_t)r0 * s.d * elt_bytes(s), st));
}

// The whole layer; s_gate/s_up/s_down non-null: the weights are E4M3 codes.
moe_status_t forward_impl(const moe_shape_t* s, const void* x, const void* w_router, const float* bias,
                          const int32_t* topk_ids_in, const float* topk_w_in, const void* w_gate, const void* w_up,
                          const void* w_down, const float* s_gate, const float* s_up, const float* s_down, void* out,
                          void* workspace, size_t ws_bytes, moe_forward_views_t* views_out, hipStream_t stream) {
  moe_status_t st = validate(s);
  if (st != MOE_OK) return st;
  if ((st = validate_gather(*s)) != MOE_OK) return st;
  if (!x || !w_gate || !w_up || !w_down || !out || !workspace) return MOE_ERR_NULL_PTR;
  if ((topk_ids_in == nullptr) != (topk_w_in == nullptr)) return MOE_ERR_INVALID_ARG;
  if (topk_ids_in == nullptr && w_router == nullptr) return MOE_ERR_NULL_PTR;
  const Plan p = make_plan(*s);
  if (ws_bytes < p.forward_ws) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return MOE_ERR_INVALID_ARG;
  char* ws = static_cast<char*>(workspace);
  moe_forward_views_t v{};
  carve(*s, p, ws + p.ws_disp, &v.disp);
  v.x_perm = nullptr;  // not materialised: the gate+up GEMM reads x through token_of
  v.h = ws + p.ws_h;
  v.y_perm = ws + p.ws_y;
  if (topk_ids_in != nullptr) {
    v.topk_ids = const_cast<int32_t*>(topk_ids_in);
    v.topk_w = const_cast<float*>(topk_w_in);
  } else {
    v.topk_ids = reinterpret_cast<int32_t*>(ws + p.ws_ids);
    v.topk_w = reinterpret_cast<float*>(ws + p.ws_w);
  }
  if (views_out != nullptr) *views_out = v;
  if (topk_ids_in == nullptr && s->T <= moe::kRouteDispatchTokens && s->E <= 64) {
    // a decode batch: routing and dispatch in one workgroup
    if (moe::launch_route_dispatch(s->dtype, x, w_router, bias, s->T, s->d, s->E, s->k, v.topk_ids, v.topk_w,
                                   small_dispatch_args(*s, p, v.topk_ids, v.disp), stream) != hipSuccess)
      return MOE_ERR_HIP;
  } else {
    if (topk_ids_in == nullptr &&
        moe::launch_route(s->dtype, x, w_router, bias, s->T, s->d, s->E, s->k, v.topk_ids, v.topk_w, stream) !=
            hipSuccess)
      return MOE_ERR_HIP;
    if ((st = enqueue_permute(*s, p, x, v.topk_ids, v.disp, nullptr, ws + p.ws_perm, stream)) != MOE_OK) return st;
  }
  // capacity mode: both passes in each launch (the overflow tiles of an expert
  // run next to its first-pass tiles and find its weights in L2)
  const int ps = s->capacity > 0 ? kBothPasses : 0;
  if ((st = enqueue_gate_up(*s, nullptr, w_gate, w_up, v.disp, ps, v.h, stream, x, s_gate, s_up)) != MOE_OK)
    return st;
  const bool split = split_down(*s, v.disp.tile_rows);
  if (fused_down_combine(*s, v.disp.tile_rows))  // a decode batch: the combine inside the down GEMM
    return enqueue_down(*s, v.h, w_down, v.disp, ps, v.y_perm, stream, s_down, true, out, v.topk_w);
  if ((st = enqueue_down(*s, v.h, w_down, v.disp, ps, v.y_perm, stream, s_down, !split)) != MOE_OK) return st;
  if (split)  // y formed from the two K ranges inside the combine
    return hip_status(moe::launch_combine_split(s->dtype, v.disp.kpart, (size_t)p.R * s->d, v.topk_w,
                                                v.disp.row_of, s->T, s->k, s->d, v.y_perm, out, stream));
  return hip_status(
      moe::launch_combine(s->dtype, v.y_perm, v.topk_w, v.disp.row_of, s->T, s->k, s->d, out, stream));
}

}  // namespace

extern "C" {

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: a shape field or size is out of range";
    case MOE_ERR_NULL_PTR: return "MOE_ERR_NULL_PTR: a required pointer is NULL";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL: workspace below the queried size";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: valid arguments the library does not implement";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a kernel launch failed";
    default: return "unknown moe_status_t";
  }
}

moe_status_t moe_query(const moe_shape_t* s, moe_sizes_t* out) {
  moe_status_t st = validate(s);
  if (st != MOE_OK) return st;
  if (out == nullptr) return MOE_ERR_NULL_PTR;
  const Plan p = make_plan(*s);
  out->rows = p.R;
  out->tile_rows = p.BM;
  out->max_tiles = (int32_t)p.max_tiles;
  out->n_passes = s->capacity > 0 ? 2 : 1;
  out->count_blocks = p.nblk;
  out->dispatch_bytes = p.dl.bytes;
  out->permute_ws_bytes = p.permute_ws;
  out->forward_ws_bytes = p.forward_ws;
  return MOE_OK;
}

moe_status_t moe_workspace_size(const moe_shape_t* s, size_t* bytes) {
  moe_status_t st = validate(s);
  if (st != MOE_OK) return st;
  if (bytes == nullptr) return MOE_ERR_NULL_PTR;
  *bytes = make_plan(*s).forward_ws;
  return MOE_OK;
}

moe_status_t moe_dispatch_carve(const moe_shape_t* s, void* base, size_t bytes, moe_dispatch_t* disp) {
  moe_status_t st = validate(s);
  if (st != MOE_OK) return st;
  if (base == nullptr || disp == nullptr) return MOE_ERR_NULL_PTR;
  const Plan p = make_plan(*s);
  if (bytes < p.dl.bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (reinterpret_cast<uintptr_t>(base) % kAlign != 0) return MOE_ERR_INVALID_ARG;
  carve(*s, p, static_cast<char*>(base), disp);
  return MOE_OK;
}

moe_status_t moe_route(const moe_shape_t* s, const void* x, const void* w_router, const float* bias,
                       int32_t* topk_ids, float* topk_w, hipStream_t stream) {
  moe_status_t st = validate(s);
  if (st != MOE_OK) return st;
  if (!x || !w_router || !topk_ids || !topk_w) return MOE_ERR_NULL_PTR;
  return hip_status(moe::launch_route(s->dtype, x, w_router, bias, s->T, s->d, s->E, s->k, topk_ids, topk_w, stream));
}

moe_status_t moe_permute(const moe_shape_t* s, const void* x, const int32_t* topk_ids, const moe_dispatch_t* disp,
                         void* x_perm, void* workspace, size_t ws_bytes, hipStream_t stream) {
  moe_status_t st = validate(s);
  if (st != MOE_OK) return st;
  if (!x || !topk_ids || !x_perm || !workspace) return MOE_ERR_NULL_PTR;
  const Plan p = make_plan(*s);
  if ((st = check_dispatch(*s, p, disp)) != MOE_OK) return st;
  if (ws_bytes < p.permute_ws) return MOE_ERR_WORKSPACE_TOO_SMALL;
  return enqueue_permute(*s, p, x, topk_ids, *disp, x_perm, workspace, stream);
}

moe_status_t moe_ffn_gate_up(const moe_shape_t* s, const void* x_perm, const void* w_gate, const void* w_up,
                             const moe_dispatch_t* disp, int pass, void* h, hipStream_t stream) {
  moe_status_t st = validate(s);
  if (st != MOE_OK) return st;
  if (!x_perm || !w_gate || !w_up || !h) return MOE_ERR_NULL_PTR;
  if (pass < 0 || pass > kBothPasses) return MOE_ERR_INVALID_ARG;
  const Plan p = make_plan(*s);
  if ((st = check_dispatch(*s, p, disp)) != MOE_OK) return st;
  return enqueue_gate_up(*s, x_perm, w_gate, w_up, *disp, pass, h, stream);
}

moe_status_t moe_ffn_gate_up_gather(const moe_shape_t* s, const void* x, const void* w_gate, const void* w_up,
                                    const moe_dispatch_t* disp, int pass, void* h, hipStream_t stream) {
  moe_status_t st = validate(s);
  if (st != MOE_OK) return st;
  if ((st = validate_gather(*s)) != MOE_OK) return st;
  if (!x || !w_gate || !w_up || !h) return MOE_ERR_NULL_PTR;
  if (pass < 0 || pass > kBothPasses) return MOE_ERR_INVALID_ARG;
  const Plan p = make_plan(*s);
  if ((st = check_dispatch(*s, p, disp)) != MOE_OK) return st;
  return enqueue_gate_up(*s, nullptr, w_gate, w_up, *disp, pass, h, stream, x);
}

moe_status_t moe_ffn_down(const moe_shape_t* s, const void* h, const void* w_down, const moe_dispatch_t* disp,
                          int pass, void* y_perm, hipStream_t stream) {
  moe_status_t st = validate(s);
  if (st != MOE_OK) return st;
  if (!h || !w_down || !y_perm) return MOE_ERR_NULL_PTR;
  if (pass < 0 || pass > kBothPasses) return MOE_ERR_INVALID_ARG;
  const Plan p = make_plan(*s);
  if ((st = check_dispatch(*s, p, disp)) != MOE_OK) return st;
  return enqueue_down(*s, h, w_down, *disp, pass, y_perm, stream);
}

moe_status_t moe_grouped_ffn(const moe_shape_t* s, const void* x_perm, const void* w_gate, const void* w_up,
                             const void* w_down, const moe_dispatch_t* disp, void* h, void* y_perm,
                             hipStream_t stream) {
  moe_status_t st = validate(s);
  if (st != MOE_OK) return st;
  if (!x_perm || !w_gate || !w_up || !w_down || !h || !y_perm) return MOE_ERR_NULL_PTR;
  const Plan p = make_plan(*s);
  if ((st = check_dispatch(*s, p, disp)) != MOE_OK) return st;
  const int passes = s->capacity > 0 ? 2 : 1;
  for (int ps = 0; ps < passes; ++ps) {
    if ((st = enqueue_gate_up(*s, x_perm, w_gate, w_up, *disp, ps, h, stream)) != MOE_OK) return st;
    if ((st = enqueue_down(*s, h, w_down, *disp, ps, y_perm, stream)) != MOE_OK) return st;
  }
  return MOE_OK;
}

moe_status_t moe_combine(const moe_shape_t* s, const void* y_perm, const float* topk_w, const moe_dispatch_t* disp,
                         void* out, hipStream_t stream) {
  moe_status_t st = validate(s);
  if (st != MOE_OK) return st;
  if (!y_perm || !topk_w || !out) return MOE_ERR_NULL_PTR;
  if (disp == nullptr) return MOE_ERR_NULL_PTR;
  if (!disp->row_of) return MOE_ERR_NULL_PTR;
  return hip_status(moe::launch_combine(s->dtype, y_perm, topk_w, disp->row_of, s->T, s->k, s->d, out, stream));
}

moe_status_t moe_forward(const moe_shape_t* s, const void* x, const void* w_router, const float* bias,
                         const int32_t* topk_ids_in, const float* topk_w_in, const void* w_gate, const void* w_up,
                         const void* w_down, void* out, void* workspace, size_t ws_bytes,
                         moe_forward_views_t* views_out, hipStream_t stream) {
  return forward_impl(s, x, w_router, bias, topk_ids_in, topk_w_in, w_gate, w_up, w_down, nullptr, nullptr,
                      nullptr, out, workspace, ws_bytes, views_out, stream);
}

moe_status_t moe_forward_noalloc(const moe_shape_t* s, const void* x, const void* w_router, const float* bias,
                                 const int32_t* topk_ids_in, const float* topk_w_in, const void* w_gate,
                                 const void* w_up, const void* w_down, void* out, moe_forward_views_t* views_out,
                                 hipStream_t stream) {
  static_assert(moe::kNoallocScratchBytes == MOE_NOALLOC_SCRATCH_BYTES, "scratch size");
  moe_status_t st = validate(s);
  if (st != MOE_OK) return st;
  if (make_plan(*s).forward_ws > moe::kNoallocScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if ((st = validate_gather(*s)) != MOE_OK) return st;
  if (!x || !w_gate || !w_up || !w_down || !out) return MOE_ERR_NULL_PTR;
  if ((topk_ids_in == nullptr) != (topk_w_in == nullptr)) return MOE_ERR_INVALID_ARG;
  if (topk_ids_in == nullptr && w_router == nullptr) return MOE_ERR_NULL_PTR;
  void* scratch = nullptr;
  if (moe::noalloc_scratch(&scratch) != hipSuccess) return MOE_ERR_HIP;
  return forward_impl(s, x, w_router, bias, topk_ids_in, topk_w_in, w_gate, w_up, w_down, nullptr, nullptr,
                      nullptr, out, scratch, moe::kNoallocScratchBytes, views_out, stream);
}

moe_status_t moe_pack_blocked16(const void* src, void* dst, int64_t matrices, int64_t rows, int64_t row_bytes,
                                hipStream_t stream) {
  if (!src || !dst) return MOE_ERR_NULL_PTR;
  if (matrices < 1 || rows < 16 || rows % 16 != 0 || row_bytes < 64 || row_bytes % 64 != 0)
    return MOE_ERR_INVALID_ARG;
  const int64_t bytes = matrices * rows * row_bytes;
  const char* a = static_cast<const char*>(src);
  const char* b = static_cast<const char*>(dst);
  if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARG;  // overlap
  if (reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe::launch_pack_blocked16(src, dst, matrices * rows / 16, row_bytes, stream));
}

moe_status_t moe_ffn_gate_up_fp8(const moe_shape_t* s, const void* x, const uint8_t* w_gate, const uint8_t* w_up,
                                 const float* s_gate, const float* s_up, const moe_dispatch_t* disp, int pass,
                                 void* h, hipStream_t stream) {
  moe_status_t st = validate(s);
  if (st != MOE_OK) return st;
  if (s->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if ((st = validate_gather(*s)) != MOE_OK) return st;
  if (!x || !w_gate || !w_up || !s_gate || !s_up || !h) return MOE_ERR_NULL_PTR;
  if (pass < 0 || pass > kBothPasses) return MOE_ERR_INVALID_ARG;
  const Plan p = make_plan(*s);
  if ((st = check_dispatch(*s, p, disp)) != MOE_OK) return st;
  return enqueue_gate_up(*s, nullptr, w_gate, w_up, *disp, pass, h, stream, x, s_gate, s_up);
}

moe_status_t moe_ffn_down_fp8(const moe_shape_t* s, const void* h, const uint8_t* w_down, const float* s_down,
                              const moe_dispatch_t* disp, int pass, void* y_perm, hipStream_t stream) {
  moe_status_t st = validate(s);
  if (st != MOE_OK) return st;
  if (s->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!h || !w_down || !s_down || !y_perm) return MOE_ERR_NULL_PTR;
  if (pass < 0 || pass > kBothPasses) return MOE_ERR_INVALID_ARG;
  const Plan p = make_plan(*s);
  if ((st = check_dispatch(*s, p, disp)) != MOE_OK) return st;
  return enqueue_down(*s, h, w_down, *disp, pass, y_perm, stream, s_down);
}

moe_status_t moe_forward_fp8(const moe_shape_t* s, const void* x, const void* w_router, const float* bias,
                             const int32_t* topk_ids_in, const float* topk_w_in, const uint8_t* w_gate,
                             const uint8_t* w_up, const uint8_t* w_down, const float* s_gate, const float* s_up,
                             const float* s_down, void* out, void* workspace, size_t ws_bytes,
                             moe_forward_views_t* views_out, hipStream_t stream) {
  moe_status_t st = validate(s);
  if (st != MOE_OK) return st;
  if (s->dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  if (!s_gate || !s_up || !s_down) return MOE_ERR_NULL_PTR;
  return forward_impl(s, x, w_router, bias, topk_ids_in, topk_w_in, w_gate, w_up, w_down, s_gate, s_up, s_down,
                      out, workspace, ws_bytes, views_out, stream);
}

}  // extern "C"
