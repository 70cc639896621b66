/*
 * Host-side checks of the C ABI's validation and planning code, built with
 * AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_abi_checked.py
 * builds the library's host code the same way).  Nothing here reaches a GPU:
 * every call either fails validation or stops at a missing pointer before the
 * first HIP call.
 *
 * For many random problem descriptions, in and out of the supported ranges:
 *  - every entry point returns a status code of moe.h (0..6);
 *  - a problem the layer accepts has a workspace that holds at least h and o
 *    of its T*k routed rows;
 *  - moe_layer and moe_layer_noalloc with a missing pointer return
 *    MOE_ERR_NULL for accepted problems and the same code as
 *    moe_layer_workspace_size otherwise;
 *  - moe_layer_plan answers as moe_layer_workspace_size does, with shape
 *    codes of moe_plan_shape_t and 1..D/64 router K slices;
 *  - status strings and stage names exist for every value, in range or not.
 * Prints "ok" and exits 0 when every check passes.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "moe.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void) {   /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}

static int32_t pick(const int32_t* v, int n) { return v[next_u32() % (uint32_t)n]; }

static int failures = 0;

#define CHECK(cond, ...)                                   \
  do {                                                     \
    if (!(cond)) {                                         \
      if (failures < 20) {                                 \
        fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
        fprintf(stderr, __VA_ARGS__);                      \
        fprintf(stderr, "\n");                             \
      }                                                    \
      ++failures;                                          \
    }                                                      \
  } while (0)

static int valid_status(moe_status_t st) { return st >= MOE_OK && st <= MOE_ERR_LAUNCH; }

/* A supported description, then (one time in three) one field replaced by a
 * value from a wider set that includes unsupported and invalid ones. */
static moe_problem_t random_problem(void) {
  static const int32_t Ts[] = {0, 1, 7, 64, 300, 512, 4097, 16384, 36000, 200000};
  static const int32_t Ds[] = {64, 128, 192, 256, 512, 1024, 2816, 4096, 8192, 16384};
  static const int32_t Es[] = {1, 3, 8, 10, 16, 64, 128, 256, 512, 1024};
  static const int32_t Is[] = {64, 128, 192, 256, 512, 704, 1024, 2048};
  static const int32_t Iss[] = {0, 64, 128, 256, 1024, 2048, 2112};
  static const int32_t wds[] = {MOE_BF16, MOE_FP8_E4M3FN, MOE_MXFP4_E2M1};
  static const int32_t wide_T[] = {-3, 0, 1, 1 << 22, 1 << 29, 0x7fffffff};
  static const int32_t wide_D[] = {-64, 0, 63, 100, 32768, 1 << 20};
  static const int32_t wide_E[] = {-1, 0, 1025, 1 << 20};
  static const int32_t wide_k[] = {-1, 0, 33, 1024};
  static const int32_t wide_I[] = {-64, 0, 32, 96, 1 << 20};
  static const int32_t wide_code[] = {-1, 3, 4, 5, 100};
  moe_problem_t p;
  memset(&p, 0, sizeof p);
  p.T = pick(Ts, sizeof Ts / sizeof *Ts);
  p.D = pick(Ds, sizeof Ds / sizeof *Ds);
  p.E = pick(Es, sizeof Es / sizeof *Es);
  p.k = 1 + (int32_t)(next_u32() % (uint32_t)(p.E < 32 ? p.E : 32));
  p.I = pick(Is, sizeof Is / sizeof *Is);
  p.I_shared = pick(Iss, sizeof Iss / sizeof *Iss);
  p.act = (int32_t)(next_u32() % 2);
  p.act_shared = (int32_t)(next_u32() % 2);
  p.renormalize = (int32_t)(next_u32() % 2);
  if (next_u32() % 6 == 0) {
    p.act_dtype = p.w_dtype = p.shared_w_dtype = MOE_F32;
  } else {
    p.act_dtype = MOE_BF16;
    p.w_dtype = pick(wds, 3);
    p.shared_w_dtype = (next_u32() % 4) ? p.w_dtype : pick(wds, 3);
  }
  p.tile_policy = (int32_t)(next_u32() % 3);
  p.act_quant = p.w_dtype == MOE_MXFP4_E2M1 ? MOE_ACT_QUANT_MXFP8
                : (p.w_dtype == MOE_FP8_E4M3FN && next_u32() % 2)
                    ? ((next_u32() % 2) ? MOE_ACT_QUANT_FP8_ROW : MOE_ACT_QUANT_FP8_SUB)
                    : MOE_ACT_QUANT_NONE;
  p.combine = (int32_t)(next_u32() % 3);
  if (next_u32() % 3 == 0) {
    switch (next_u32() % 12) {
      case 0: p.T = pick(wide_T, 6); break;
      case 1: p.D = pick(wide_D, 6); break;
      case 2: p.E = pick(wide_E, 4); break;
      case 3: p.k = pick(wide_k, 4); break;
      case 4: p.I = pick(wide_I, 5); break;
      case 5: p.I_shared = pick(wide_I, 5); break;
      case 6: p.act = pick(wide_code, 5); break;
      case 7: p.act_dtype = pick(wide_code, 5); break;
      case 8: p.w_dtype = pick(wide_code, 5); break;
      case 9: p.tile_policy = pick(wide_code, 5); break;
      case 10: p.act_quant = pick(wide_code, 5); break;
      default: p.combine = pick(wide_code, 5); break;
    }
  }
  return p;
}

int main(void) {
  const int N = 20000;
  int accepted = 0;
  for (int it = 0; it < N; ++it) {
    moe_problem_t p = random_problem();
    size_t ws = 0;
    moe_status_t st = moe_layer_workspace_size(&p, &ws);
    CHECK(valid_status(st), "layer workspace status %d", (int)st);
    if (st == MOE_OK) {
      ++accepted;
      /* the workspace holds at least h and o of the routed rows */
      const size_t a = p.act_dtype == MOE_F32 ? 4 : 2;
      const size_t lower = (size_t)p.T * (size_t)p.k * ((size_t)p.I + (size_t)p.D) * a;
      CHECK(ws >= lower, "workspace %zu below the routed rows' h and o (%zu)", ws, lower);
    }
    /* a missing pointer: the layer's own answer, before any device work */
    moe_layer_args_t args;
    memset(&args, 0, sizeof args);
    moe_status_t sl = moe_layer(&p, &args, NULL, 0, NULL);
    CHECK(valid_status(sl), "layer status %d", (int)sl);
    CHECK(sl == (st == MOE_OK ? MOE_ERR_NULL : st), "moe_layer %d vs workspace %d", (int)sl, (int)st);
    moe_status_t sn = moe_layer_noalloc(&p, NULL, NULL);
    CHECK(sn == (st == MOE_OK ? MOE_ERR_NULL : st), "noalloc %d vs workspace %d", (int)sn, (int)st);
    /* the plan: the same answer as the workspace, codes in range */
    moe_plan_t plan;
    memset(&plan, 0xff, sizeof plan);
    moe_status_t sq = moe_layer_plan(&p, &plan);
    CHECK(sq == st, "plan %d vs workspace %d", (int)sq, (int)st);
    CHECK(moe_layer_plan(&p, NULL) == (st == MOE_OK ? MOE_ERR_NULL : st), "plan with null out");
    if (sq == MOE_OK) {
      CHECK(plan.router >= MOE_PLAN_STREAM_16 && plan.router <= MOE_PLAN_TILED_32x64 &&
                plan.gate_up >= MOE_PLAN_STREAM_16 && plan.gate_up <= MOE_PLAN_TILED_32x64 &&
                plan.down >= MOE_PLAN_STREAM_16 && plan.down <= MOE_PLAN_TILED_32x64,
            "plan codes %d %d %d", (int)plan.router, (int)plan.gate_up, (int)plan.down);
      CHECK(plan.router_slices >= 1 && plan.router_slices <= p.D / 64, "router slices %d", (int)plan.router_slices);
      CHECK(plan.one_launch_permute == 0 || plan.one_launch_permute == 1, "permute flag");
    }

    size_t pws = 0;
    moe_status_t sp = moe_permute_workspace_size(&p, &pws);
    CHECK(valid_status(sp), "permute workspace status %d", (int)sp);
    int32_t ng = (int32_t)(next_u32() % 1100) - 20, rub = (int32_t)(next_u32() % 400000) - 50;
    size_t fws = 0;
    moe_status_t sf = moe_grouped_ffn_workspace_size(&p, ng, rub, &fws);
    CHECK(valid_status(sf), "grouped ffn workspace status %d", (int)sf);
    moe_status_t sr = moe_route(&p, NULL, NULL, NULL, 0, NULL, NULL, NULL);
    CHECK(valid_status(sr) && sr != MOE_OK, "route with null pointers: %d", (int)sr);
    moe_status_t sc = moe_combine(&p, NULL, NULL, NULL, NULL, NULL, NULL);
    CHECK(valid_status(sc) && (sc != MOE_OK || p.T == 0), "combine with null pointers: %d", (int)sc);
  }
  /* null problem and null outputs */
  size_t ws = 0;
  CHECK(moe_layer_workspace_size(NULL, &ws) == MOE_ERR_NULL, "null problem");
  moe_problem_t ok;
  memset(&ok, 0, sizeof ok);
  ok.T = 64; ok.D = 256; ok.E = 8; ok.k = 2; ok.I = 128; ok.renormalize = 1;
  ok.act_dtype = MOE_F32; ok.w_dtype = MOE_F32; ok.shared_w_dtype = MOE_F32;
  CHECK(moe_layer_workspace_size(&ok, &ws) == MOE_OK && ws > 0, "reference problem accepted");
  CHECK(moe_layer_workspace_size(&ok, NULL) == MOE_ERR_NULL, "null size output");
  /* quantiser argument checks */
  for (int it = 0; it < 2000; ++it) {
    int32_t rows = (int32_t)(next_u32() % 100) - 5, cols = (int32_t)(next_u32() % 40000) - 8;
    int64_t lda = (int64_t)cols + (int64_t)(next_u32() % 64) - 16;
    moe_status_t s1 = moe_quantize_rows(NULL, rows, cols, lda, NULL, NULL, NULL);
    moe_status_t s2 = moe_quantize_rows_mx(NULL, rows, cols, lda, NULL, NULL, NULL);
    moe_status_t s3 = moe_quantize_subchannel(NULL, rows, cols, lda, NULL, NULL, NULL);
    CHECK(valid_status(s1) && valid_status(s2) && valid_status(s3), "quantiser status %d %d %d", (int)s1,
          (int)s2, (int)s3);
    CHECK(rows != 0 || s1 != MOE_ERR_NULL, "zero rows need no pointers");
  }
  /* names of every value */
  for (int v = -5; v < 12; ++v) CHECK(moe_status_string((moe_status_t)v) != NULL, "status string %d", v);
  for (int v = -3; v < moe_stage_count() + 3; ++v) CHECK(moe_stage_name(v) != NULL, "stage name %d", v);
  double ms[2];
  int32_t cnt[2];
  moe_status_t tr = moe_timing_read(ms, cnt, 2);
  CHECK(valid_status(tr), "timing read status %d", (int)tr);
  CHECK(moe_layer_noalloc_max_bytes() > 0, "noalloc size");
  if (failures) {
    fprintf(stderr, "%d failures over %d problems (%d accepted)\n", failures, N, accepted);
    return 1;
  }
  printf("ok: %d problems, %d accepted\n", N, accepted);
  return 0;
}
