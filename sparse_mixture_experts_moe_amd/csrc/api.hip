// C ABI of the MoE layer: validation, workspace planning, tile policy, launch
// order and per-stage event timing.  See include/moe.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <vector>

#include "../../include/moe.h"
#include "moe_kernels.h"

using namespace moe;

namespace {

constexpr size_t ALIGN = 256;
size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

size_t dt_bytes(int dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : 1; }

bool act_ok(int a) { return a == MOE_ACT_SILU || a == MOE_ACT_GELU_TANH; }
bool dt_ok(int d) { return d == MOE_F32 || d == MOE_BF16 || d == MOE_FP8_E4M3FN; }
bool wdt_ok(int d) { return dt_ok(d) || d == MOE_MXFP4_E2M1; }

bool combo_ok(int act_dt, int w_dt) {
  if (act_dt == MOE_F32) return w_dt == MOE_F32;
  if (act_dt == MOE_BF16) return w_dt == MOE_BF16 || w_dt == MOE_FP8_E4M3FN || w_dt == MOE_MXFP4_E2M1;
  return false;
}

bool quantised(const moe_problem_t* p) { return p->act_quant != MOE_ACT_QUANT_NONE; }

// Bytes of the activation scales of `rows` quantised rows of `cols` columns:
// one fp32 per row, (sub-channel) one fp32 per 512 columns, or (MXFP8) one
// E8M0 byte per 32 columns.
size_t qscale_bytes(const moe_problem_t* p, int64_t rows, int64_t cols) {
  if (p->act_quant == MOE_ACT_QUANT_FP8_SUB) return static_cast<size_t>(rows * (cols / kSubChannel) * 4);
  return static_cast<size_t>(p->act_quant == MOE_ACT_QUANT_MXFP8 ? rows * (cols / 32) : rows * 4);
}

// Device dtype of the expert GEMMs' activations.
int gemm_a_dtype(const moe_problem_t* p) {
  return p->act_quant == MOE_ACT_QUANT_FP8_ROW ? DT_FP8
         : p->act_quant == MOE_ACT_QUANT_FP8_SUB ? DT_FP8S
         : p->act_quant == MOE_ACT_QUANT_MXFP8 ? DT_MXFP8 : p->act_dtype;
}

// Quantise `rows` bf16 rows with the problem's activation quantisation.
hipError_t quant_rows(const moe_problem_t* p, const void* a, int rows, int cols, uint8_t* q,
                      void* scale, hipStream_t s) {
  if (p->act_quant == MOE_ACT_QUANT_MXFP8)
    return launch_quant_rows_mx(static_cast<const uint16_t*>(a), rows, cols, cols, q,
                                static_cast<uint8_t*>(scale), s);
  if (p->act_quant == MOE_ACT_QUANT_FP8_SUB)
    return launch_quant_rows_sub(static_cast<const uint16_t*>(a), rows, cols, cols, q,
                                 static_cast<float*>(scale), s);
  return launch_quant_rows(static_cast<const uint16_t*>(a), rows, cols, cols, q,
                           static_cast<float*>(scale), s);
}

// Point a GEMM set's activation and weight scales at the right buffers (S.K
// set first: the sub-channel scales' last slice is the epilogue's).
void set_scales(const moe_problem_t* p, GSet& S, const void* a_scale, int32_t a_scale_rows,
                const void* w_scale, int w_dtype, int64_t w_scale_gstride_bytes) {
  S.a_scale = nullptr;
  S.a_mx = nullptr;
  S.w_mx = nullptr;
  S.scale = nullptr;
  S.a_sub = nullptr;
  if (p->act_quant == MOE_ACT_QUANT_FP8_ROW) S.a_scale = static_cast<const float*>(a_scale);
  if (p->act_quant == MOE_ACT_QUANT_FP8_SUB) {
    S.a_sub = static_cast<const float*>(a_scale);
    S.a_sub_rows = a_scale_rows;
    S.a_scale = S.a_sub + static_cast<int64_t>(S.K / kSubChannel - 1) * a_scale_rows;
  }
  if (p->act_quant == MOE_ACT_QUANT_MXFP8) {
    S.a_mx = static_cast<const uint8_t*>(a_scale);
    S.a_mx_rows = a_scale_rows;
  }
  if (w_dtype == MOE_FP8_E4M3FN) S.scale = static_cast<const float*>(w_scale);
  if (w_dtype == MOE_MXFP4_E2M1) {
    S.w_mx = static_cast<const uint8_t*>(w_scale);
    S.w_mx_gstride = w_scale_gstride_bytes;
  }
}

// weights that need a scale argument
bool w_scaled(int w_dtype) { return w_dtype == MOE_FP8_E4M3FN || w_dtype == MOE_MXFP4_E2M1; }

// Checks common to every entry point.
bool tiled_fits(const moe_problem_t* p);

moe_status_t check_problem(const moe_problem_t* p, bool need_ffn, bool need_router) {
  if (!p) return MOE_ERR_NULL;
  if (p->T < 0 || p->D <= 0 || p->D % 64 || p->E < 1 || p->E > 1024) return MOE_ERR_SHAPE;
  if (need_router && (p->k < 1 || p->k > 32 || p->k > p->E)) return MOE_ERR_SHAPE;
  if (need_ffn && (p->I <= 0 || p->I % 64 || p->I_shared < 0 || p->I_shared % 64))
    return MOE_ERR_SHAPE;
  // Row indices are int32 (T*k rows); element offsets are 64-bit everywhere
  // except the LDS-tiled GEMM's per-lane byte offsets, which the plan checks
  // (tiled_fits: bf16 layers fall back to the register-streamed GEMM, the
  // quantised modes, tiled only, are refused below).
  const int64_t Tk = static_cast<int64_t>(p->T) * std::max(p->k, 1);
  if (Tk >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  // launch grids are int32: row tiles (16 rows at the least, routed and
  // shared) times column blocks (64 columns at the least) stay below 2^31
  const int64_t wide = std::max<int64_t>({p->D, p->I, p->I_shared, p->E});
  if ((Tk / 16 + p->T / 16 + p->E + 2) * (wide / 64 + 1) >= (int64_t(1) << 31)) return MOE_ERR_SHAPE;
  if (!dt_ok(p->act_dtype) || !wdt_ok(p->w_dtype) || !wdt_ok(p->shared_w_dtype)) return MOE_ERR_DTYPE;
  if (!act_ok(p->act) || !act_ok(p->act_shared)) return MOE_ERR_DTYPE;
  if (p->tile_policy < MOE_TILE_AUTO || p->tile_policy > MOE_TILE_LDS) return MOE_ERR_DTYPE;
  if (p->act_dtype == MOE_FP8_E4M3FN) return MOE_ERR_UNSUPPORTED;
  if (need_ffn && !combo_ok(p->act_dtype, p->w_dtype)) return MOE_ERR_UNSUPPORTED;
  if (need_ffn && p->I_shared && !combo_ok(p->act_dtype, p->shared_w_dtype))
    return MOE_ERR_UNSUPPORTED;
  if (p->renormalize != 0 && p->renormalize != 1) return MOE_ERR_UNSUPPORTED;
  if (p->act_quant < MOE_ACT_QUANT_NONE || p->act_quant > MOE_ACT_QUANT_FP8_SUB) return MOE_ERR_UNSUPPORTED;
  if (p->combine < MOE_COMBINE_AUTO || p->combine > MOE_COMBINE_FUSED) return MOE_ERR_UNSUPPORTED;
  // MXFP4 weights go with MXFP8 activations and nothing else, on both branches
  const bool mx = p->act_quant == MOE_ACT_QUANT_MXFP8;
  if (need_ffn && (mx != (p->w_dtype == MOE_MXFP4_E2M1) ||
                   (p->I_shared && mx != (p->shared_w_dtype == MOE_MXFP4_E2M1))))
    return MOE_ERR_UNSUPPORTED;
  if (need_ffn && quantised(p)) {
    // fp8 x fp8 and MXFP8 x MXFP4 run on the tiled kernel only, with one
    // weight format on both branches
    const int wdt = mx ? MOE_MXFP4_E2M1 : MOE_FP8_E4M3FN;
    if (p->act_dtype != MOE_BF16 || p->w_dtype != wdt) return MOE_ERR_UNSUPPORTED;
    if (p->I_shared && p->shared_w_dtype != wdt) return MOE_ERR_UNSUPPORTED;
    if (p->tile_policy == MOE_TILE_STREAM) return MOE_ERR_UNSUPPORTED;
    const int km = p->act_quant == MOE_ACT_QUANT_FP8_SUB ? kSubChannel : tiled_k_multiple_a8();
    if (p->D % km || p->I % km || p->I_shared % km) return MOE_ERR_UNSUPPORTED;
    const int qm = quant_max_cols();
    if (p->D > qm || p->I > qm || p->I_shared > qm) return MOE_ERR_UNSUPPORTED;
    if (!tiled_fits(p)) return MOE_ERR_SHAPE;
  }
  return MOE_OK;
}

// ---------------------------------------------------------------- tile policy
struct Plan {
  bool tiled;  // LDS-tiled kernel
  int mt;      // stream kernel: 16-row chunks per m-tile
  int bm;      // rows per m-tile
  int shape;   // tiled kernel: TILED_TALL / TILED_SMALL / TILED_WIDE, or -1 = wide /
               // narrow picked per launch
};

constexpr bool kTiledReady = true;

// Tile policy thresholds on the mean rows per group (the measured choices):
//  - streamed GEMM: 16-row tiles up to kStream16Mean, 32-row up to
//    kStream32Mean, 64-row beyond;
//  - LDS-tiled GEMM: the 32-row shape for decode-sized groups (up to
//    kSmallMax; fp8 weights above kSmallMin, since below it the streamed
//    kernel's 16-row tiles read fewer padded rows), 256-row tiles up to
//    kTallMean (an expert's weights are read once per 256 rows), 128-row
//    tiles beyond.
constexpr double kStream16Mean = 4.0;
constexpr double kStream32Mean = 24.0;
constexpr double kSmallMin = 8.0;
constexpr double kSmallMax = 48.0;
constexpr double kTallMean = 192.0;

// The tiled GEMM's 32-bit offsets cover every operand of the expert FFNs.
bool tiled_fits(const moe_problem_t* p) {
  const int64_t T = p->T, Tk = T * p->k, D = p->D, I = p->I, Is = p->I_shared;
  const int km = tiled_k_multiple();
  if (D % km || I % km || Is % km) return false;
  return tiled_offsets_fit(T, D, 2 * I, D, p->w_dtype) && tiled_offsets_fit(Tk, I, D, I, p->w_dtype) &&
         (!Is || (tiled_offsets_fit(T, D, 2 * Is, D, p->shared_w_dtype) &&
                  tiled_offsets_fit(T, Is, D, Is, p->shared_w_dtype)));
}

Plan make_plan(const moe_problem_t* p, double mean_rows) {
  if (quantised(p)) {
    // fp8 x fp8, MXFP8 x MXFP4: the tiled kernel's quantised shapes (with
    // sub-channel scales, no 128 x 512 tiles)
    const bool wide_ok = p->act_quant != MOE_ACT_QUANT_FP8_SUB;
    const int shape = mean_rows <= kSmallMax ? TILED_SMALLQ
                      : (mean_rows <= kTallMean || !wide_ok) ? TILED_TALL : TILED_WIDE;
    return Plan{true, 0, tiled_bm(shape), shape};
  }
  const bool tiled_ok = kTiledReady && p->act_dtype == MOE_BF16 && tiled_fits(p);
  int policy = p->tile_policy;
  const int ks = tiled_k_multiple_small();
  const bool small_bf16 = p->w_dtype == MOE_BF16 && (!p->I_shared || p->shared_w_dtype == MOE_BF16) &&
                          mean_rows <= kSmallMax;
  const bool small_fp8 = p->w_dtype == MOE_FP8_E4M3FN &&
                         (!p->I_shared || p->shared_w_dtype == MOE_FP8_E4M3FN) &&
                         mean_rows > kSmallMin && mean_rows <= kSmallMax;
  if (policy == MOE_TILE_AUTO && tiled_ok && (small_fp8 || small_bf16) &&
      p->D % ks == 0 && p->I % ks == 0 && p->I_shared % ks == 0)
    return Plan{true, 0, tiled_bm(TILED_SMALL), TILED_SMALL};
  if (policy == MOE_TILE_AUTO) policy = (tiled_ok && mean_rows > 48.0) ? MOE_TILE_LDS : MOE_TILE_STREAM;
  if (policy == MOE_TILE_LDS && tiled_ok) {
    // 256-row tiles read an expert's weights half as often; measured faster
    // while groups average a few hundred rows at most, 128-row tiles beyond
    if (mean_rows <= kTallMean) return Plan{true, 0, tiled_bm(TILED_TALL), TILED_TALL};
    return Plan{true, 0, tiled_bm(TILED_WIDE), -1};
  }
  int mt = mean_rows <= kStream16Mean ? 1 : mean_rows <= kStream32Mean ? 2 : 4;
  mt = std::min(mt, stream_max_mt(p->act_dtype));
  return Plan{false, mt, 16 * mt, -1};
}

// Down projection of the fused layer.  Where gate/up runs on 256-row tiles
// (bf16, up to kTallMean rows per expert), the down projection takes 128-row
// tiles from a tile table of its own (128 x 512 blocks, or 128 x 256 where
// those pad D less): its K is I rather than D, so a 256-row tile's blocks are
// short, and 128-row blocks measured faster there (Qwen prefill down
// projection 1.74 -> 1.64 ms; Gemma, D = 2816 on 128 x 256 blocks, 0.211 ->
// 0.202 ms) while gate/up keeps the 256-row tiles.
// Under the 32-row decode tiles with bf16 weights, the down projection takes
// 64-wide weight blocks on the same M-tile table (twice the blocks; Qwen decode
// down projection 0.501 -> 0.487 ms).
Plan down_plan(const moe_problem_t* p, const Plan& up) {
  if (up.tiled && up.shape == TILED_TALL && !quantised(p))
    return Plan{true, 0, tiled_bm(TILED_WIDE), -1};
  if (up.tiled && up.shape == TILED_SMALL && p->w_dtype == MOE_BF16 &&
      (!p->I_shared || p->shared_w_dtype == MOE_BF16))
    return Plan{true, 0, tiled_bm(TILED_SMALLD), TILED_SMALLD};
  return up;
}

int routed_tile_ub(int64_t rows, int groups, int bm) {
  return static_cast<int>(std::min<int64_t>(groups, rows) + rows / bm);
}

int blocks_per_m(const Plan& pl, int shape, bool gated, int n_out) {
  if (pl.tiled) return tiled_blocks_n(shape, gated, n_out);
  return (stream_waves_n(gated, n_out) + 3) / 4;
}

// Dense tiled launches (128-row tiles) use the wide block (512 weight rows)
// unless the narrow one (256) pads the output columns of the launch's sets less.
int pick_dense_shape(const GArgs& g, bool gated) {
  int64_t pad_w = 0, pad_n = 0;
  for (int i = 0; i < g.nsets; ++i) {
    const int n = g.s[i].n_out, ww = gated ? 256 : 512, wn = gated ? 128 : 256;
    pad_w += static_cast<int64_t>(tiled_blocks_n(TILED_WIDE, gated, n)) * ww - n;
    pad_n += static_cast<int64_t>(tiled_blocks_n(TILED_NARROW, gated, n)) * wn - n;
  }
  return pad_w <= pad_n ? TILED_WIDE : TILED_NARROW;
}

void finish_grid(GArgs& g, const Plan& pl, bool gated) {
  int b = 0;
  g.shape = !pl.tiled ? -1 : pl.shape >= 0 ? pl.shape : pick_dense_shape(g, gated);
  for (int i = 0; i < g.nsets; ++i) {
    GSet& S = g.s[i];
    S.blocks_per_m = blocks_per_m(pl, g.shape, gated, S.n_out);
    S.block0 = b;
    S.bm = pl.bm;
    b += S.m_slots * S.blocks_per_m * std::max(1, S.ksplit);
  }
  g.total_blocks = b;
}

// The router is one dense group of T rows.  From kRouterTiledT tokens (and E
// a multiple of 4: the tiled GEMM stores four output columns at a time) it
// runs on the LDS-tiled GEMM; below (decode), on the streamed GEMM with the K
// dimension split into slices whose fp32 partial sums the top-k kernel adds in
// slice order, so enough wavefronts stream the router weight.  From
// kRouterTallT tokens with E a multiple of 256 it takes 256-row tiles (one
// block per CU): every weight tile is copied by half as many row tiles.
// Measured: Ling prefill (16384 tokens) router 122 -> 108 us, Qwen prefill
// (8192 tokens) 64 -> 56 us, against 128-row tiles.
constexpr int kRouterTiledT = 512;   // measured: Ling decode router 28 -> 20.5 us vs 1024
constexpr int kRouterTallT = 4096;
Plan router_plan(const moe_problem_t* p) {
  if (kTiledReady && p->act_dtype == MOE_BF16 && p->T >= kRouterTallT && p->E % 256 == 0 &&
      p->tile_policy != MOE_TILE_STREAM && p->D % tiled_k_multiple() == 0 &&
      tiled_offsets_fit(p->T, p->D, p->E, p->D, p->act_dtype))
    return Plan{true, 0, tiled_bm(TILED_TALL), TILED_TALL};
  if (kTiledReady && p->act_dtype == MOE_BF16 && p->T >= kRouterTiledT &&
      p->tile_policy != MOE_TILE_STREAM && p->E % 4 == 0 &&
      p->D % tiled_k_multiple() == 0 && tiled_offsets_fit(p->T, p->D, p->E, p->D, p->act_dtype))
    return Plan{true, 0, tiled_bm(TILED_WIDE), -1};
  int mt = p->T <= 16 ? 1 : p->T <= 32 ? 2 : 4;
  mt = std::min(mt, stream_max_mt(p->act_dtype));
  return Plan{false, mt, 16 * mt, -1};
}

// K slices of the router: the most slices (a divisor of D / 64) that keeps
// each slice at least kRouterSlice long and the work items (tiled blocks or
// stream wavefronts) at most kRouterItems (one round of blocks: half as many
// for 256-row tiles, one per CU).  Measured: finer splits make the router
// faster and top-k slower by as much (more partial sums to add).
constexpr int kRouterSlice = 256;
constexpr int kRouterItems = 512;
int router_splits(const moe_problem_t* p, const Plan& pl) {
  const int64_t m_tiles = (static_cast<int64_t>(p->T) + pl.bm - 1) / pl.bm;
  const bool tall = pl.tiled && pl.shape == TILED_TALL;
  const int64_t items = pl.tiled ? m_tiles * tiled_blocks_n(tall ? TILED_TALL : TILED_NARROW, false, p->E)
                                 : m_tiles * stream_waves_n(false, p->E);
  const int64_t max_items = tall ? kRouterItems / 2 : kRouterItems;
  const int K = p->D;
  int s = 1;
  for (int c = 2; c <= K / 64; ++c)
    if ((K / 64) % c == 0 && K / c >= kRouterSlice && items * c <= max_items) s = c;
  return s;
}

hipError_t run_gemm(const GArgs& g, const Plan& pl, bool gated, int a_dt, int w_dt, int o_dt,
                    hipStream_t s) {
  if (pl.tiled) return launch_tiled_gemm(g, g.shape, gated, w_dt, o_dt, a_dt, s);
  if (a_dt == DT_FP8 || a_dt == DT_MXFP8) return hipErrorInvalidValue;
  return launch_stream_gemm(g, pl.mt, gated, a_dt, w_dt, o_dt, s);
}

// ---------------------------------------------------------------- timing
enum Stage { ST_ROUTER = 0, ST_TOPK, ST_PERMUTE, ST_TILES, ST_FFN1, ST_FFN2, ST_COMBINE, ST_QUANT,
             ST_COUNT };
const char* kStageNames[ST_COUNT] = {"router_gemm", "topk_softmax", "permute", "tile_table",
                                     "ffn1_gate_up_act", "ffn2_down", "combine", "act_quant"};

struct TimingRec {
  int stage;
  hipEvent_t a, b;
};
// The timing record belongs to the calling host thread (the library's only
// state; see moe_timing_enable).
thread_local bool g_timing = false;
thread_local bool g_no_events = false;   // set while moe_layer_noalloc runs: no event creation
thread_local uint32_t g_timing_mask = 0xffffffffu;   // stages timed while g_timing
thread_local std::vector<TimingRec> g_recs;
thread_local std::vector<hipEvent_t> g_pool;

hipEvent_t take_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct StageScope {
  int stage;
  hipStream_t s;
  hipEvent_t a = nullptr;
  StageScope(int st, hipStream_t st_s) : stage(st), s(st_s) {
    if (g_timing && !g_no_events && ((g_timing_mask >> st) & 1u) && (a = take_event()) &&
        hipEventRecord(a, s) != hipSuccess) {
      g_pool.push_back(a);
      a = nullptr;
    }
  }
  ~StageScope() {
    if (!a) return;
    hipEvent_t b = take_event();
    if (!b) {
      g_pool.push_back(a);
      return;
    }
    if (hipEventRecord(b, s) != hipSuccess) {
      g_pool.push_back(a);
      g_pool.push_back(b);
      return;
    }
    g_recs.push_back(TimingRec{stage, a, b});
  }
};

#define MOE_LAUNCH(expr)                                   \
  do {                                                     \
    if ((expr) != hipSuccess) return MOE_ERR_LAUNCH;       \
  } while (0)

// ---------------------------------------------------------------- workspace layouts
struct Carve {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

// Arrival counters of the fused combine: one per token and N block of the
// down projection, sized for the narrowest tiled block (64 output columns).
int64_t fused_max_nb(const moe_problem_t* p) { return (p->D + 63) / 64; }

// The permutation and the M-tile table run as one single-block launch for
// small batches under the decode-sized (or streamed) plans.
bool one_launch_permute(const moe_problem_t* p, const Plan& pl) {
  return p->T <= perm_small_max_tokens() &&
         (!pl.tiled || pl.shape == TILED_SMALL || pl.shape == TILED_SMALLQ);
}

struct LayerLayout {
  size_t logits, idx, w, counts, offsets, row_token, row_of_slot, blk, rank, tiles, ntiles;
  size_t tiles2, ntiles2;            // the down projection's own tile table (when plan2 differs)
  size_t h, h_sh, o, o_sh, cnt, total;
  size_t xq, sx, hq, sh, hsq, shs;   // quantised activations and their scales (act_quant)
  int tile_ub, tile_ub2;
  int splits;
  Plan plan, plan2;
};

LayerLayout layer_layout(const moe_problem_t* p) {
  LayerLayout L{};
  const int64_t T = p->T, Tk = T * p->k, E = p->E;
  const size_t a = dt_bytes(p->act_dtype);
  L.plan = make_plan(p, E ? static_cast<double>(Tk) / E : 0.0);
  L.tile_ub = routed_tile_ub(Tk, p->E, L.plan.bm);
  L.plan2 = down_plan(p, L.plan);
  L.tile_ub2 = routed_tile_ub(Tk, p->E, L.plan2.bm);
  Carve c;
  L.splits = router_splits(p, router_plan(p));
  L.logits = c.take(T * E * 4 * L.splits);
  L.idx = c.take(Tk * 4);
  L.w = c.take(Tk * 4);
  L.counts = c.take(E * 4);
  L.offsets = c.take((E + 1) * 4);
  L.row_token = c.take(Tk * 4);
  L.row_of_slot = c.take(Tk * 4);
  L.blk = c.take(static_cast<size_t>(perm_blocks(p->T)) * E * 4);
  L.rank = c.take(Tk * 4);
  L.tiles = c.take(static_cast<size_t>(L.tile_ub) * sizeof(GTile));
  L.ntiles = c.take(16);
  if (L.plan2.bm != L.plan.bm) {
    L.tiles2 = c.take(static_cast<size_t>(L.tile_ub2) * sizeof(GTile));
    L.ntiles2 = c.take(16);
  } else {
    L.tiles2 = L.tiles;
    L.ntiles2 = L.ntiles;
  }
  L.h = c.take(Tk * p->I * a);
  L.h_sh = c.take(T * p->I_shared * a);
  L.o = c.take(Tk * p->D * a);
  L.o_sh = c.take(p->I_shared ? T * p->D * a : 0);
  L.cnt = c.take(T * fused_max_nb(p) * 4);
  if (quantised(p)) {
    L.xq = c.take(T * p->D);
    L.sx = c.take(qscale_bytes(p, T, p->D));
    L.hq = c.take(Tk * p->I);
    L.sh = c.take(qscale_bytes(p, Tk, p->I));
    L.hsq = c.take(T * p->I_shared);
    L.shs = c.take(qscale_bytes(p, T, p->I_shared));
  }
  L.total = c.off;
  return L;
}

struct PermLayout {
  size_t blk, rank, total;
};
PermLayout perm_layout(const moe_problem_t* p) {
  PermLayout L{};
  Carve c;
  L.blk = c.take(static_cast<size_t>(perm_blocks(p->T)) * p->E * 4);
  L.rank = c.take(static_cast<size_t>(p->T) * p->k * 4);
  L.total = c.off;
  return L;
}

// Workspace of moe_grouped_ffn: the M-tile table, and with fp8 activations the
// quantised A rows (gathered or not: sized for both) and h with their scales.
struct FfnLayout {
  size_t tiles, ntiles, aq, sa, hq, sh, total;
};
FfnLayout ffn_layout(const moe_problem_t* p, const Plan& pl, int n_groups, int rows_ub) {
  FfnLayout L{};
  Carve c;
  L.tiles = c.take(static_cast<size_t>(routed_tile_ub(rows_ub, n_groups, pl.bm)) * sizeof(GTile));
  L.ntiles = c.take(16);
  if (quantised(p)) {
    const int64_t a_rows = std::max(p->T, rows_ub);
    L.aq = c.take(static_cast<size_t>(a_rows) * p->D);
    L.sa = c.take(qscale_bytes(p, a_rows, p->D));
    L.hq = c.take(static_cast<size_t>(rows_ub) * p->I);
    L.sh = c.take(qscale_bytes(p, rows_ub, p->I));
  }
  L.total = c.off;
  return L;
}

// router product through the plain (ungated) grouped GEMM: one dense group,
// written as `splits` partial sums part[s][T][E].
hipError_t launch_router(const moe_problem_t* p, const void* x, const void* wr, float* part,
                         int splits, hipStream_t s) {
  const Plan pl = router_plan(p);
  GArgs g{};
  g.nsets = 1;
  GSet& S = g.s[0];
  S.K = p->D;
  S.a_rows = p->T;
  S.a = x;
  S.lda = p->D;
  S.w = wr;
  S.NB = p->E;
  S.n_out = p->E;
  S.out = part;
  S.ldo = p->E;
  S.rows = p->T;
  S.m_slots = static_cast<int32_t>((static_cast<int64_t>(p->T) + pl.bm - 1) / pl.bm);
  S.ksplit = splits;
  S.split_stride = static_cast<int64_t>(p->T) * p->E;
  finish_grid(g, pl, false);
  return run_gemm(g, pl, false, p->act_dtype, p->act_dtype, MOE_F32, s);
}

}  // namespace

// ====================================================================== ABI
extern "C" {

const char* moe_status_string(moe_status_t st) {
  // C callers may pass any int: read the bits rather than the enum value
  // (a C++ enum holding a value outside its range is undefined)
  int32_t v;
  std::memcpy(&v, &st, sizeof v);
  switch (v) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "null pointer";
    case MOE_ERR_SHAPE: return "size out of the supported range";
    case MOE_ERR_DTYPE: return "unknown dtype, activation or policy code";
    case MOE_ERR_UNSUPPORTED: return "unsupported combination";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_LAUNCH: return "kernel launch or HIP runtime call failed";
  }
  return "unknown status";
}

moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* w_router, float* logits,
                       int32_t logits_given, int32_t* topk_idx, float* topk_w, void* stream) {
  moe_status_t st = check_problem(p, false, true);
  if (st != MOE_OK) return st;
  if (!logits || !topk_idx || !topk_w || (!logits_given && (!x || !w_router))) return MOE_ERR_NULL;
  if (p->act_dtype == MOE_FP8_E4M3FN) return MOE_ERR_UNSUPPORTED;
  if (p->T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!logits_given) {
    // no workspace here: the router writes whole sums straight into `logits`
    StageScope sc(ST_ROUTER, s);
    MOE_LAUNCH(launch_router(p, x, w_router, logits, 1, s));
  }
  StageScope sc(ST_TOPK, s);
  MOE_LAUNCH(launch_topk_softmax(logits, 1, nullptr, p->T, p->E, p->k, p->renormalize, topk_idx,
                                 topk_w, s));
  return MOE_OK;
}

moe_status_t moe_permute_workspace_size(const moe_problem_t* p, size_t* bytes) {
  moe_status_t st = check_problem(p, false, true);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_NULL;
  *bytes = perm_layout(p).total;
  return MOE_OK;
}

moe_status_t moe_permute(const moe_problem_t* p, const int32_t* topk_idx, int32_t* counts,
                         int32_t* offsets, int32_t* row_token, int32_t* row_of_slot, const void* x,
                         void* x_perm, void* ws, size_t ws_bytes, void* stream) {
  moe_status_t st = check_problem(p, false, true);
  if (st != MOE_OK) return st;
  if (!topk_idx || !counts || !offsets || !row_token || !row_of_slot) return MOE_ERR_NULL;
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_NULL;
  if (x && (reinterpret_cast<uintptr_t>(x) % 16 || reinterpret_cast<uintptr_t>(x_perm) % 16))
    return MOE_ERR_SHAPE;
  const PermLayout L = perm_layout(p);
  if (L.total && !ws) return MOE_ERR_NULL;
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (p->T == 0) return MOE_OK;
  char* w = static_cast<char*>(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  StageScope sc(ST_PERMUTE, s);
  if (p->T <= perm_small_max_tokens()) {
    MOE_LAUNCH(launch_permute_small(topk_idx, p->T, p->k, p->E, counts, offsets, row_token,
                                    row_of_slot, 1, 0, false, nullptr, nullptr, s));
  } else {
    MOE_LAUNCH(launch_permute(topk_idx, p->T, p->k, p->E, reinterpret_cast<int32_t*>(w + L.blk),
                              reinterpret_cast<int32_t*>(w + L.rank), counts, offsets, row_token,
                              row_of_slot, s));
  }
  if (x)
    MOE_LAUNCH(launch_gather_rows(x, row_token, offsets + p->E, p->T, p->T * p->k,
                                  static_cast<int64_t>(p->D) * dt_bytes(p->act_dtype), x_perm, s));
  return MOE_OK;
}

moe_status_t moe_grouped_ffn_workspace_size(const moe_problem_t* p, int32_t n_groups,
                                            int32_t rows_upper_bound, size_t* bytes) {
  moe_status_t st = check_problem(p, true, false);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_NULL;
  if (n_groups < 1 || n_groups > 1024 || rows_upper_bound < 0) return MOE_ERR_SHAPE;
  // the A rows, h and out hold rows_upper_bound rows: the same element bound
  // as the layer's T*k rows (the tiled GEMM's 32-bit byte offsets)
  if (static_cast<int64_t>(rows_upper_bound) * std::max(p->D, p->I) >= (int64_t(1) << 31))
    return MOE_ERR_SHAPE;
  const Plan pl = make_plan(p, static_cast<double>(rows_upper_bound) / n_groups);
  *bytes = ffn_layout(p, pl, n_groups, rows_upper_bound).total;
  return MOE_OK;
}

moe_status_t moe_grouped_ffn(const moe_problem_t* p, int32_t n_groups, int32_t rows_upper_bound,
                             const void* a, const int32_t* row_token, const int32_t* offsets,
                             const void* w13, const void* s13, const void* w2, const void* s2,
                             void* h, void* out, void* ws, size_t ws_bytes, void* stream) {
  size_t need = 0;
  moe_status_t st = moe_grouped_ffn_workspace_size(p, n_groups, rows_upper_bound, &need);
  if (st != MOE_OK) return st;
  if (!a || !offsets || !w13 || !w2 || !h || !out || !ws) return MOE_ERR_NULL;
  if (w_scaled(p->w_dtype) && (!s13 || !s2)) return MOE_ERR_NULL;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (rows_upper_bound == 0) return MOE_OK;
  const Plan pl = make_plan(p, static_cast<double>(rows_upper_bound) / n_groups);
  const int tile_ub = routed_tile_ub(rows_upper_bound, n_groups, pl.bm);
  const FfnLayout FL = ffn_layout(p, pl, n_groups, rows_upper_bound);
  char* w = static_cast<char*>(ws);
  GTile* tiles = reinterpret_cast<GTile*>(w + FL.tiles);
  int32_t* ntiles = reinterpret_cast<int32_t*>(w + FL.ntiles);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool aq = quantised(p);
  const int a_dt = gemm_a_dtype(p);
  const int a_rows = row_token ? p->T : rows_upper_bound;
  if (row_token && p->T <= 0) return MOE_ERR_SHAPE;
  uint8_t* aq8 = reinterpret_cast<uint8_t*>(w + FL.aq);
  void* sa = w + FL.sa;
  uint8_t* hq = reinterpret_cast<uint8_t*>(w + FL.hq);
  void* sh = w + FL.sh;
  if (aq) {
    StageScope sc(ST_QUANT, s);
    MOE_LAUNCH(quant_rows(p, a, a_rows, p->D, aq8, sa, s));
  }
  {
    StageScope sc(ST_TILES, s);
    MOE_LAUNCH(launch_build_tiles(offsets, n_groups, pl.bm, rows_upper_bound, tile_ub, pl.tiled,
                                  tiles, ntiles, s));
  }
  GArgs g1{};
  g1.nsets = 1;
  {
    GSet& S = g1.s[0];
    S.K = p->D;
    S.a_rows = a_rows;
    S.a = aq ? static_cast<const void*>(aq8) : a;
    S.gather = row_token;
    S.lda = p->D;
    S.w = w13;
    set_scales(p, S, sa, a_rows, s13, p->w_dtype, static_cast<int64_t>(p->D / 128) * 2 * p->I * 4);
    S.w_gstride = static_cast<int64_t>(2) * p->I * p->D;
    S.s_gstride = 2 * p->I;
    S.NB = 2 * p->I;
    S.n_out = p->I;
    S.act = p->act;
    S.out = h;
    S.ldo = p->I;
    S.tiles = tiles;
    S.n_tiles = ntiles;
    S.m_slots = tile_ub;
  }
  finish_grid(g1, pl, true);
  GArgs g2 = g1;
  {
    GSet& S = g2.s[0];
    S.K = p->I;
    S.a_rows = rows_upper_bound;
    S.a = aq ? static_cast<void*>(hq) : h;
    S.gather = nullptr;
    S.lda = p->I;
    S.w = w2;
    set_scales(p, S, sh, rows_upper_bound, s2, p->w_dtype, static_cast<int64_t>(p->I / 128) * p->D * 4);
    S.w_gstride = static_cast<int64_t>(p->D) * p->I;
    S.s_gstride = p->D;
    S.NB = p->D;
    S.n_out = p->D;
    S.out = out;
    S.ldo = p->D;
  }
  finish_grid(g2, pl, false);
  {
    StageScope sc(ST_FFN1, s);
    MOE_LAUNCH(run_gemm(g1, pl, true, a_dt, p->w_dtype, p->act_dtype, s));
  }
  if (aq) {
    StageScope sc(ST_QUANT, s);
    MOE_LAUNCH(quant_rows(p, h, rows_upper_bound, p->I, hq, sh, s));
  }
  {
    StageScope sc(ST_FFN2, s);
    MOE_LAUNCH(run_gemm(g2, pl, false, a_dt, p->w_dtype, p->act_dtype, s));
  }
  return MOE_OK;
}

moe_status_t moe_combine(const moe_problem_t* p, const void* o_perm, const int32_t* row_of_slot,
                         const float* topk_w, const void* shared_out, void* y, void* stream) {
  moe_status_t st = check_problem(p, false, true);
  if (st != MOE_OK) return st;
  if (!o_perm || !row_of_slot || !topk_w || !y) return MOE_ERR_NULL;
  if (p->act_dtype == MOE_FP8_E4M3FN) return MOE_ERR_UNSUPPORTED;
  if (p->T == 0) return MOE_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  StageScope sc(ST_COMBINE, s);
  MOE_LAUNCH(launch_combine(o_perm, row_of_slot, topk_w, shared_out, p->T, p->D, p->k,
                            p->act_dtype, y, s));
  return MOE_OK;
}

}  // extern "C"

namespace {

// The layer's problem and the pointers it requires.
moe_status_t check_layer_args(const moe_problem_t* p, const moe_layer_args_t* A) {
  moe_status_t st = check_problem(p, true, true);
  if (st != MOE_OK) return st;
  if (!A || !A->x || !A->w13 || !A->w2 || !A->y) return MOE_ERR_NULL;
  if (!A->logits_in && !A->w_router) return MOE_ERR_NULL;
  if (w_scaled(p->w_dtype) && (!A->s13 || !A->s2)) return MOE_ERR_NULL;
  if (p->I_shared) {
    if (!A->w13_shared || !A->w2_shared) return MOE_ERR_NULL;
    if (w_scaled(p->shared_w_dtype) && (!A->s13_shared || !A->s2_shared)) return MOE_ERR_NULL;
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_layer_workspace_size(const moe_problem_t* p, size_t* bytes) {
  moe_status_t st = check_problem(p, true, true);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_NULL;
  *bytes = layer_layout(p).total;
  return MOE_OK;
}

moe_status_t moe_layer_plan(const moe_problem_t* p, moe_plan_t* out) {
  moe_status_t st = check_problem(p, true, true);
  if (st != MOE_OK) return st;
  if (!out) return MOE_ERR_NULL;
  const LayerLayout L = layer_layout(p);
  // a plan's shape as the launch resolves it: the dense 128-row tiles take the
  // wide or the narrow block per launch (the sets it covers, as moe_layer
  // groups them: one launch per weight dtype)
  const bool split_sets = p->w_dtype != p->shared_w_dtype && p->I_shared;
  auto code = [&](const Plan& pl, bool gated, int n_shared, int n_routed) -> int32_t {
    if (!pl.tiled) return pl.mt == 1 ? MOE_PLAN_STREAM_16 : pl.mt == 2 ? MOE_PLAN_STREAM_32 : MOE_PLAN_STREAM_64;
    int shape = pl.shape;
    if (shape < 0) {
      GArgs g{};
      if (n_shared > 0 && !split_sets) g.s[g.nsets++].n_out = n_shared;
      g.s[g.nsets++].n_out = n_routed;
      shape = pick_dense_shape(g, gated);
    }
    switch (shape) {
      case TILED_TALL: return MOE_PLAN_TILED_256x256;
      case TILED_WIDE: return MOE_PLAN_TILED_128x512;
      case TILED_NARROW: return MOE_PLAN_TILED_128x256;
      case TILED_SMALL: return MOE_PLAN_TILED_32x128;
      case TILED_SMALLQ: return MOE_PLAN_TILED_64x256;
      case TILED_SMALLD:
      default: return MOE_PLAN_TILED_32x64;
    }
  };
  const Plan rp = router_plan(p);
  out->router = code(rp, false, 0, p->E);
  out->router_slices = L.splits;
  out->gate_up = code(L.plan, true, p->I_shared, p->I);
  out->down = code(L.plan2, false, p->I_shared ? p->D : 0, p->D);
  out->one_launch_permute = one_launch_permute(p, L.plan);
  return MOE_OK;
}

moe_status_t moe_layer(const moe_problem_t* p, const moe_layer_args_t* A, void* ws, size_t ws_bytes,
                       void* stream) {
  moe_status_t st = check_layer_args(p, A);
  if (st != MOE_OK) return st;
  const LayerLayout L = layer_layout(p);
  if (!ws) return MOE_ERR_NULL;
  if (ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (p->T == 0) return MOE_OK;

  char* w = static_cast<char*>(ws);
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto pick = [&](auto* user, size_t off) {
    using Ptr = decltype(user);
    return user ? user : reinterpret_cast<Ptr>(w + off);
  };
  // router partial sums (or whole logits when not split), then top-k
  float* part = A->logits_in ? const_cast<float*>(A->logits_in)
                : (L.splits == 1 ? pick(A->logits_out, L.logits) : reinterpret_cast<float*>(w + L.logits));
  const int splits = A->logits_in ? 1 : L.splits;
  float* logits_write = (A->logits_out && part != A->logits_out) ? A->logits_out : nullptr;
  int32_t* idx = pick(A->topk_idx_out, L.idx);
  float* tw = pick(A->topk_w_out, L.w);
  int32_t* counts = pick(A->counts_out, L.counts);
  int32_t* offsets = pick(A->offsets_out, L.offsets);
  int32_t* row_token = pick(A->row_token_out, L.row_token);
  int32_t* row_of_slot = pick(A->row_of_slot_out, L.row_of_slot);
  GTile* tiles = reinterpret_cast<GTile*>(w + L.tiles);
  int32_t* ntiles = reinterpret_cast<int32_t*>(w + L.ntiles);
  void* h = w + L.h;
  void* h_sh = w + L.h_sh;
  void* o = w + L.o;
  void* o_sh = w + L.o_sh;
  const int64_t Tk = static_cast<int64_t>(p->T) * p->k;
  const Plan& pl = L.plan;
  const Plan& pl2 = L.plan2;
  GTile* tiles2 = reinterpret_cast<GTile*>(w + L.tiles2);
  int32_t* ntiles2 = reinterpret_cast<int32_t*>(w + L.ntiles2);

  // 1. router logits (fp32) and top-k softmax
  if (!A->logits_in) {
    StageScope sc(ST_ROUTER, s);
    MOE_LAUNCH(launch_router(p, A->x, A->w_router, part, L.splits, s));
  }
  {
    StageScope sc(ST_TOPK, s);
    MOE_LAUNCH(launch_topk_softmax(part, splits, logits_write, p->T, p->E, p->k, p->renormalize,
                                   idx, tw, s));
  }
  // 2. permutation and the M-tile table (one launch for small batches)
  if (one_launch_permute(p, pl)) {
    StageScope sc(ST_PERMUTE, s);
    MOE_LAUNCH(launch_permute_small(idx, p->T, p->k, p->E, counts, offsets, row_token, row_of_slot,
                                    pl.bm, L.tile_ub, pl.tiled, tiles, ntiles, s));
  } else {
    {
      StageScope sc(ST_PERMUTE, s);
      MOE_LAUNCH(launch_permute(idx, p->T, p->k, p->E, reinterpret_cast<int32_t*>(w + L.blk),
                                reinterpret_cast<int32_t*>(w + L.rank), counts, offsets, row_token,
                                row_of_slot, s));
    }
    {
      StageScope sc(ST_TILES, s);
      if (tiles2 != tiles)   // both tables share the order (both plans are tiled)
        MOE_LAUNCH(launch_build_tiles_pair(offsets, p->E, static_cast<int>(Tk), pl.tiled, pl.bm,
                                           L.tile_ub, tiles, ntiles, pl2.bm, L.tile_ub2, tiles2,
                                           ntiles2, s));
      else
        MOE_LAUNCH(launch_build_tiles(offsets, p->E, pl.bm, static_cast<int>(Tk), L.tile_ub,
                                      pl.tiled, tiles, ntiles, s));
    }
  }
  // 3. grouped FFN: shared branch (dense rows) and routed experts in the same launches
  // quantised activations: x quantised once, h per row after the gate/up GEMM
  const bool aq = quantised(p);
  const int a_dt = gemm_a_dtype(p);
  uint8_t* xq = reinterpret_cast<uint8_t*>(w + L.xq);
  void* sx = w + L.sx;
  uint8_t* hq = reinterpret_cast<uint8_t*>(w + L.hq);
  void* sh = w + L.sh;
  uint8_t* hsq = reinterpret_cast<uint8_t*>(w + L.hsq);
  void* shs = w + L.shs;
  if (aq) {
    StageScope sc(ST_QUANT, s);
    MOE_LAUNCH(quant_rows(p, A->x, p->T, p->D, xq, sx, s));
  }
  GArgs g1{};
  int si = 0;
  if (p->I_shared) {
    GSet& S = g1.s[si++];
    S.K = p->D;
    S.a_rows = p->T;
    S.a = aq ? static_cast<const void*>(xq) : A->x;
    S.lda = p->D;
    S.w = A->w13_shared;
    set_scales(p, S, sx, p->T, A->s13_shared, p->shared_w_dtype, 0);
    S.NB = 2 * p->I_shared;
    S.n_out = p->I_shared;
    S.act = p->act_shared;
    S.out = h_sh;
    S.ldo = p->I_shared;
    S.rows = p->T;
    S.m_slots = static_cast<int32_t>((static_cast<int64_t>(p->T) + pl.bm - 1) / pl.bm);
  }
  {
    GSet& S = g1.s[si++];
    S.K = p->D;
    S.a_rows = p->T;
    S.a = aq ? static_cast<const void*>(xq) : A->x;
    S.gather = row_token;
    S.lda = p->D;
    S.w = A->w13;
    set_scales(p, S, sx, p->T, A->s13, p->w_dtype, static_cast<int64_t>(p->D / 128) * 2 * p->I * 4);
    S.w_gstride = static_cast<int64_t>(2) * p->I * p->D;
    S.s_gstride = 2 * p->I;
    S.NB = 2 * p->I;
    S.n_out = p->I;
    S.act = p->act;
    S.out = h;
    S.ldo = p->I;
    S.tiles = tiles;
    S.n_tiles = ntiles;
    S.m_slots = L.tile_ub;
  }
  g1.nsets = si;
  finish_grid(g1, pl, true);
  GArgs g2 = g1;
  si = 0;
  if (p->I_shared) {
    GSet& S = g2.s[si++];
    S.K = p->I_shared;
    S.a_rows = p->T;
    S.a = aq ? static_cast<void*>(hsq) : h_sh;
    S.lda = p->I_shared;
    S.w = A->w2_shared;
    set_scales(p, S, shs, p->T, A->s2_shared, p->shared_w_dtype, 0);
    S.NB = p->D;
    S.n_out = p->D;
    S.out = o_sh;
    S.ldo = p->D;
    S.m_slots = static_cast<int32_t>((static_cast<int64_t>(p->T) + pl2.bm - 1) / pl2.bm);
  }
  {
    GSet& S = g2.s[si++];
    S.K = p->I;
    S.a_rows = static_cast<int32_t>(Tk);
    S.a = aq ? static_cast<void*>(hq) : h;
    S.gather = nullptr;
    S.lda = p->I;
    S.w = A->w2;
    set_scales(p, S, sh, static_cast<int32_t>(Tk), A->s2, p->w_dtype, static_cast<int64_t>(p->I / 128) * p->D * 4);
    S.w_gstride = static_cast<int64_t>(p->D) * p->I;
    S.s_gstride = p->D;
    S.NB = p->D;
    S.n_out = p->D;
    S.out = o;
    S.ldo = p->D;
    S.tiles = tiles2;
    S.n_tiles = ntiles2;
    S.m_slots = L.tile_ub2;
  }
  finish_grid(g2, pl2, false);
  bool fused = false;
  if (p->w_dtype != p->shared_w_dtype && p->I_shared) {
    // one launch covers one weight dtype: run the two sets separately
    for (int i = 0; i < 2; ++i) {
      GArgs a1{}, a2{};
      a1.nsets = a2.nsets = 1;
      a1.s[0] = g1.s[i];
      a2.s[0] = g2.s[i];
      finish_grid(a1, pl, true);
      finish_grid(a2, pl2, false);
      const int wdt = i == 0 ? p->shared_w_dtype : p->w_dtype;
      {
        StageScope sc(ST_FFN1, s);
        MOE_LAUNCH(run_gemm(a1, pl, true, p->act_dtype, wdt, p->act_dtype, s));
      }
      {
        StageScope sc(ST_FFN2, s);
        MOE_LAUNCH(run_gemm(a2, pl2, false, p->act_dtype, wdt, p->act_dtype, s));
      }
    }
  } else {
    {
      StageScope sc(ST_FFN1, s);
      MOE_LAUNCH(run_gemm(g1, pl, true, a_dt, p->w_dtype, p->act_dtype, s));
    }
    if (aq) {
      StageScope sc(ST_QUANT, s);
      MOE_LAUNCH(quant_rows(p, h, static_cast<int>(Tk), p->I, hq, sh, s));
      if (p->I_shared) MOE_LAUNCH(quant_rows(p, h_sh, p->T, p->I_shared, hsq, shs, s));
    }
    // 4a. the combine inside the down projection (owner computes; see moe.h)
    const int nb = g2.s[g2.nsets - 1].blocks_per_m;
    // (MOE_COMBINE_AUTO keeps the separate combine: measured faster on every
    // layer here, e.g. Ling decode 2.41 vs 2.53 ms, Ling prefill 14.4 vs 16.8 ms)
    fused = p->combine == MOE_COMBINE_FUSED && pl2.tiled && p->act_dtype == MOE_BF16 &&
            nb <= fused_max_nb(p);
    for (int i = 0; i < g2.nsets; ++i) fused = fused && g2.s[i].ksplit <= 1 && g2.s[i].blocks_per_m == nb;
    if (fused) {
      GFuse& F = g2.fc;
      F.cnt = reinterpret_cast<int32_t*>(w + L.cnt);
      F.row_of_slot = row_of_slot;
      F.w = tw;
      F.o = o;
      F.o_sh = p->I_shared ? o_sh : nullptr;
      F.y = A->y;
      F.T = p->T;
      F.D = p->D;
      F.k = p->k;
      F.nb = nb;
      F.expect = p->k + (p->I_shared ? 1 : 0);
      g2.s[g2.nsets - 1].out_token = row_token;   // the routed set (the shared set's rows are tokens)
    }
    {
      StageScope sc(ST_FFN2, s);
      if (fused) MOE_LAUNCH(launch_fill_i32(g2.fc.cnt, static_cast<int64_t>(p->T) * nb, 0, s));
      MOE_LAUNCH(run_gemm(g2, pl2, false, a_dt, p->w_dtype, p->act_dtype, s));
    }
  }
  // 4. unpermute + weighted combine + shared branch (unless fused above)
  if (!fused) {
    StageScope sc(ST_COMBINE, s);
    MOE_LAUNCH(launch_combine(o, row_of_slot, tw, p->I_shared ? o_sh : nullptr, p->T, p->D, p->k,
                              p->act_dtype, A->y, s));
  }
  return MOE_OK;
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free layer
// For callers that cannot allocate (code under graph capture, tight serving
// loops): moe_layer_noalloc runs moe_layer with its workspace in a fixed
// device array instead of a caller buffer.  The host side names the array
// only in hipGetSymbolAddress: each device holds its own copy at its own
// address, taken once per device with that device current, and that address
// is what the kernels receive.
namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The scratch array's address on device `dev` (nullptr on failure).
void* scratch_on(int dev) {
  std::call_once(g_scratch_once[dev], [dev] {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_err[dev] = e;
    g_scratch_ptr[dev] = e == hipSuccess ? ptr : nullptr;
    if (cur >= 0 && cur != dev) (void)hipSetDevice(cur);
  });
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t moe_layer_noalloc_max_bytes(void) { return kScratchBytes; }

moe_status_t moe_layer_noalloc(const moe_problem_t* p, const moe_layer_args_t* A, void* stream) {
  moe_status_t st = check_layer_args(p, A);   // before any HIP call
  if (st != MOE_OK) return st;
  size_t need = 0;
  st = moe_layer_workspace_size(p, &need);
  if (st != MOE_OK) return st;
  if (need > kScratchBytes) return MOE_ERR_WORKSPACE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = -1;
  if (hipStreamGetDevice(s, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_LAUNCH;
  void* ws = scratch_on(dev);
  if (!ws) return MOE_ERR_LAUNCH;
  g_no_events = true;
  st = moe_layer(p, A, ws, kScratchBytes, stream);
  g_no_events = false;
  return st;
}

moe_status_t moe_quantize_rows(const void* a, int32_t rows, int32_t cols, int64_t lda, uint8_t* q,
                               float* scale, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 8 || cols > quant_max_cols() || lda < cols || lda % 8)
    return MOE_ERR_SHAPE;
  if (rows == 0) return MOE_OK;
  if (!a || !q || !scale) return MOE_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(a) % 16 || reinterpret_cast<uintptr_t>(q) % 8) return MOE_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  StageScope sc(ST_QUANT, s);
  MOE_LAUNCH(launch_quant_rows(static_cast<const uint16_t*>(a), rows, cols, lda, q, scale, s));
  return MOE_OK;
}

moe_status_t moe_quantize_rows_mx(const void* a, int32_t rows, int32_t cols, int64_t lda, uint8_t* q,
                                  uint8_t* scale, void* stream) {
  if (rows < 0 || cols <= 0 || cols % 128 || cols > quant_max_cols() || lda < cols || lda % 8)
    return MOE_ERR_SHAPE;
  if (rows == 0) return MOE_OK;
  if (!a || !q || !scale) return MOE_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(a) % 16 || reinterpret_cast<uintptr_t>(q) % 8) return MOE_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  StageScope sc(ST_QUANT, s);
  MOE_LAUNCH(launch_quant_rows_mx(static_cast<const uint16_t*>(a), rows, cols, lda, q, scale, s));
  return MOE_OK;
}

moe_status_t moe_quantize_subchannel(const void* a, int32_t rows, int32_t cols, int64_t lda, uint8_t* q,
                                     float* scale, void* stream) {
  if (rows < 0 || cols <= 0 || cols % kSubChannel || cols > quant_max_cols() || lda < cols || lda % 8)
    return MOE_ERR_SHAPE;
  if (rows == 0) return MOE_OK;
  if (!a || !q || !scale) return MOE_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(a) % 16 || reinterpret_cast<uintptr_t>(q) % 8) return MOE_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  StageScope sc(ST_QUANT, s);
  MOE_LAUNCH(launch_quant_rows_sub(static_cast<const uint16_t*>(a), rows, cols, lda, q, scale, s));
  return MOE_OK;
}

// ---------------------------------------------------------------- timing ABI
moe_status_t moe_timing_enable(int32_t on) {
  g_timing = on != 0;
  g_timing_mask = on >= 0 ? 0xffffffffu : static_cast<uint32_t>(on) & 0x7fffffffu;
  return MOE_OK;
}

moe_status_t moe_timing_read(double* ms, int32_t* launches, int32_t n_stages) {
  if ((!ms || !launches) && n_stages > 0) return MOE_ERR_NULL;
  moe_status_t st = MOE_OK;
  for (const TimingRec& r : g_recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
      st = MOE_ERR_LAUNCH;
    if (r.stage < n_stages) {
      ms[r.stage] += t;
      launches[r.stage] += 1;
    }
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  return st;
}

int32_t moe_stage_count(void) { return ST_COUNT; }

const char* moe_stage_name(int32_t stage) {
  return (stage >= 0 && stage < ST_COUNT) ? kStageNames[stage] : "unknown";
}

moe_status_t moe_probe_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return MOE_ERR_NULL;
  if (bytes <= 0 || bytes % 16 || reinterpret_cast<uintptr_t>(buf) % 16) return MOE_ERR_SHAPE;
  MOE_LAUNCH(launch_probe_hbm_read(buf, bytes, sink, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

int32_t moe_probe_mfma_sink_floats(void) { return probe_mfma_threads(); }

moe_status_t moe_probe_mfma(int32_t dtype, const void* operands, int32_t iters, float* sink,
                            double* flop, void* stream) {
  if (!operands || !sink || !flop) return MOE_ERR_NULL;
  if (dtype != MOE_BF16 && dtype != MOE_FP8_E4M3FN) return MOE_ERR_DTYPE;
  if (iters <= 0 || reinterpret_cast<uintptr_t>(operands) % 16) return MOE_ERR_SHAPE;
  MOE_LAUNCH(launch_probe_mfma(dtype == MOE_FP8_E4M3FN, operands, iters, sink, flop,
                               static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status_t moe_debug_fp8_to_bf16(const uint8_t* codes, uint16_t* out, int32_t n, void* stream) {
  if (!codes || !out) return MOE_ERR_NULL;
  if (n < 0 || n % 8) return MOE_ERR_SHAPE;
  MOE_LAUNCH(launch_fp8_decode(codes, out, n, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status_t moe_debug_f32_to_fp8(const float* v, uint8_t* out, int32_t n, void* stream) {
  if (!v || !out) return MOE_ERR_NULL;
  if (n < 0 || n % 2) return MOE_ERR_SHAPE;
  MOE_LAUNCH(launch_fp8_encode(v, out, n, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

}  // extern "C"
