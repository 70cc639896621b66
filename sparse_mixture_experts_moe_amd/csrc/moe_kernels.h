// Internal declarations shared by the HIP sources of the MoE library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ------------------------------------------------------------------ dtypes
// DT_MXFP4: e2m1 pairs per byte (element 2j in the low nibble) with E8M0
// block scales; DT_MXFP8: e4m3fn codes with E8M0 block scales (activations);
// DT_FP8S: e4m3fn codes with one fp32 scale per kSubChannel-element slice of
// a row (activations)
enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_MXFP4 = 3, DT_MXFP8 = 4, DT_FP8S = 5 };
constexpr int kSubChannel = 512;
enum : int { ACT_SILU = 0, ACT_GELU_TANH = 1 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));   // 16 raw bytes in registers

// bf16 storage is handled as raw uint16_t.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// ------------------------------------------------------------------ grouped GEMM
// One M-tile of a group: sorted rows [row0, row1) of group `group`.
struct GTile {
  int32_t group;
  int32_t row0;
  int32_t row1;
  int32_t pad;
};

// A set of groups sharing one weight tensor (routed experts, or the shared
// branch as a single group).  Rows are numbered inside the set.
struct GSet {
  int32_t K;                // reduction length (D for gate/up, I for down)
  int32_t a_rows;           // rows of the A storage (gathered rows are checked against it)
  const void* a;            // A storage, row stride lda elements
  const int32_t* gather;    // A row of set row r = gather ? gather[r] : r
  int64_t lda;
  const float* a_scale;     // fp8 A: per-A-row (storage row) dequantisation scale
  // MX block scales (E8M0 bytes; per group of 128 K elements, a row's four
  // block scales side by side): A rows [K/128][a_mx_rows][4] (storage rows),
  // weights [groups][K/128][NB][4]
  const uint8_t* a_mx;
  int32_t a_mx_rows;
  const uint8_t* w_mx;
  int64_t w_mx_gstride;     // bytes between groups' weight scales
  // sub-channel scales of fp8 A rows (DT_FP8S): [K / kSubChannel][a_sub_rows]
  // fp32 (storage rows); a_scale then points at the last slice's row of them
  const float* a_sub;
  int32_t a_sub_rows;
  const void* w;            // [groups][NB][K] weight storage
  const float* scale;       // [groups][NB] per-output-channel scales or null
  int64_t w_gstride;        // elements between groups (NB*K)
  int64_t s_gstride;        // scale elements between groups (NB)
  int32_t NB;               // weight rows: 2*I (gated) or N (plain)
  int32_t n_out;            // output columns: I (gated) or N (plain)
  int32_t act;              // gated activation
  void* out;                // output storage, row stride ldo elements
  int64_t ldo;
  const GTile* tiles;       // m-tile table, or null for dense tiles over [0, rows)
  const int32_t* n_tiles;   // device count of valid table entries
  int32_t rows;             // dense: number of rows
  int32_t m_slots;          // m-tile slots the grid reserves for this set
  int32_t block0;           // first block id of this set
  int32_t blocks_per_m;     // blocks per m-tile slot (N direction)
  int32_t bm;               // rows per m-tile
  int32_t ksplit;           // K slices (>1 only for plain fp32 outputs: partial sums)
  int64_t split_stride;     // output elements between the partial sums of two slices
  const int32_t* out_token; // fused combine: token of output row r (null: r itself)
};

// Combine fused into the down projection (bf16 rows, tiled kernel, no K
// slices): after a block has stored its output rows, each row adds one to
// the arrival counter of (its token, the block's N block).  The block whose
// addition completes a counter (expect arrivals: the token's k routed rows
// and its shared row) owns that token's columns of the N block: it sums the
// token's rows exactly as the separate combine does (fp32, slot order, the
// shared row last, one rounding) and writes y.  The owner is whichever block
// arrives last, but the sum does not depend on it, so y is bit-identical to
// the separate combine's.
struct GFuse {
  int32_t* cnt;                // [T][nb] arrival counters, zero at launch; null: no fused combine
  const int32_t* row_of_slot;  // [T*k] routed row of slot (t, j)
  const float* w;              // [T*k] routing weight of slot (t, j)
  const void* o;               // [T*k][D] routed rows
  const void* o_sh;            // [T][D] shared rows, or null
  void* y;                     // [T][D]
  int32_t T, D, k;
  int32_t nb;                  // N blocks of the launch (counters per token)
  int32_t expect;              // arrivals per (token, N block)
};

struct GArgs {
  GSet s[2];
  int32_t nsets;
  int32_t total_blocks;
  int32_t shape;            // tiled kernel: TILED_* block shape (host-side choice)
  GFuse fc;
};

// ------------------------------------------------------------------ device helpers
// fp8 e4m3fn -> bf16 is exact (every e4m3fn value is a bf16 value):
// v_cvt_scalef32_pk_bf16_fp8 with scale 1 converts two codes per instruction.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(lo), 1.0f, false);
  const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(lo), 1.0f, true);
  const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(hi), 1.0f, false);
  const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(hi), 1.0f, true);
  bf16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

// Operand of one MFMA step (8 K-elements per lane) from staged uint4s.
template <int DT>
__device__ __forceinline__ bf16x8 operand_bf16(const uint4* v, int u) {
  if constexpr (DT == DT_BF16) {
    return __builtin_bit_cast(bf16x8, v[u]);
  } else {  // DT_FP8: 8 bytes of step u
    const uint4 q = v[u >> 1];
    return (u & 1) ? fp8x8_to_bf16x8(q.z, q.w) : fp8x8_to_bf16x8(q.x, q.y);
  }
}

__device__ __forceinline__ float act_fn(int act, float z) {
  if (act == ACT_SILU) return z / (1.0f + expf(-z));
  const float c = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * z * (1.0f + tanhf(c * (z + 0.044715f * z * z * z)));
}

// Which set / M-tile / N-block a block works on; false if it has no work.
__device__ __forceinline__ bool resolve_block(const GArgs& g, int b, int& si, int& group, int& row0,
                                              int& row1, int& nblk) {
  si = (g.nsets > 1 && b >= g.s[1].block0) ? 1 : 0;
  const GSet& S = g.s[si];
  int local = b - S.block0;
  if (S.ksplit > 1) local /= S.ksplit;
  // consecutive blocks: same tile, consecutive N blocks
  const int m = local / S.blocks_per_m;
  nblk = local - m * S.blocks_per_m;
  if (S.tiles) {
    if (m >= S.n_tiles[0]) return false;
    const GTile t = S.tiles[m];
    group = t.group;
    row0 = t.row0;
    row1 = t.row1;
  } else {
    row0 = m * S.bm;
    if (row0 >= S.rows) return false;
    row1 = min(row0 + S.bm, S.rows);
    group = 0;
  }
  return row1 > row0;
}

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error.

// Router logits given as `splits` partial sums part[s][T][E] (fp32), added in
// slice order -> topk idx / weights; the summed logits are written to
// logits_out when it is not null.
// renorm 1: weights renormalised over the k selected; 0: plain softmax probabilities.
hipError_t launch_topk_softmax(const float* part, int splits, float* logits_out, int T, int E,
                               int k, int renorm, int32_t* idx, float* w, hipStream_t s);

// Permutation: per-block bit masks -> counts/offsets -> stable scatter.
int perm_blocks(int T);
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* blk /*[nb*E]*/,
                          int32_t* local_rank /*[T*k]*/, int32_t* counts, int32_t* offsets,
                          int32_t* row_token, int32_t* row_of_slot, hipStream_t s);

// x_perm[r] = x[row_token[r]] (row_bytes, a multiple of 16, per row) for the
// rows r < min(rows, *n_rows) (n_rows: device pointer, offsets[E]); rows whose
// token is outside [0, T) are left as they are.
hipError_t launch_gather_rows(const void* x, const int32_t* row_token, const int32_t* n_rows, int T,
                              int rows, int64_t row_bytes, void* x_perm, hipStream_t s);

// Batches of at most perm_small_max_tokens() tokens: permutation and, when
// tiles is not null, the M-tile table (group order or, spread, a fixed order
// that puts neighbouring groups far apart) in one single-block launch.
int perm_small_max_tokens();
hipError_t launch_permute_small(const int32_t* idx, int T, int k, int E, int32_t* counts,
                                int32_t* offsets, int32_t* row_token, int32_t* row_of_slot, int bm,
                                int max_tiles, bool spread, GTile* tiles, int32_t* n_tiles,
                                hipStream_t s);

// M-tile table of n_groups groups from device offsets, in group order or, with
// largest_first, by descending group size (ties by group id).  Offsets are
// clamped to [0, max_rows] and at most max_tiles entries are written.
hipError_t launch_build_tiles(const int32_t* offsets, int n_groups, int bm, int max_rows,
                              int max_tiles, bool largest_first, GTile* tiles, int32_t* n_tiles,
                              hipStream_t s);
// Two tables of the same groups in the same order in one launch: bm-row tiles
// (at most max_tiles) and bm2-row tiles (at most max_tiles2).
hipError_t launch_build_tiles_pair(const int32_t* offsets, int n_groups, int max_rows,
                                   bool largest_first, int bm, int max_tiles, GTile* tiles,
                                   int32_t* n_tiles, int bm2, int max_tiles2, GTile* tiles2,
                                   int32_t* n_tiles2, hipStream_t s);

// Grouped GEMM, streamed weights.  mt = 16-row chunks per m-tile (1, 2, 4).
// gated: h = act(A.Wg^T * sg) * (A.Wu^T * su); plain: out = A.W^T * s.
// a_dtype / w_dtype / out_dtype: DT_*.
hipError_t launch_stream_gemm(const GArgs& g, int mt, bool gated, int a_dtype, int w_dtype,
                              int out_dtype, hipStream_t s);
int stream_waves_n(bool gated, int n_out);   // wave tiles along N per m-tile
int stream_max_mt(int a_dtype);              // largest mt the stream kernel runs for a dtype

// Grouped GEMM, LDS-tiled (bf16 activations, bf16 or fp8 weights).  Block
// shapes (rows x weight rows): TILED_TALL 256 x 256 (expert FFNs), TILED_WIDE
// 128 x 512 and TILED_NARROW 128 x 256 (two blocks per CU), TILED_SMALL
// 32 x 128 (two blocks per CU; decode-sized groups), TILED_SMALLQ 64 x 256
// (two blocks per CU; decode-sized groups with fp8 or MXFP8 activations),
// TILED_SMALLD 32 x 64 (the ungated bf16-weight product of decode-sized
// groups: the down projection).  Every set's bm must be tiled_bm(shape).
enum : int { TILED_TALL = 0, TILED_WIDE = 1, TILED_NARROW = 2, TILED_SMALL = 3, TILED_SMALLQ = 4,
             TILED_SMALLD = 5 };
// a_dtype DT_FP8 (fp8 activations with fp8 weights, bf16 output, one block
// per CU shapes only) needs every set's a_scale; DT_FP8S (the same with
// sub-channel scales, K a multiple of kSubChannel, no K slices) every set's
// a_sub, a_sub_rows >= a_rows, and a_scale at the last slice; a_dtype DT_MXFP8 (with
// DT_MXFP4 weights, same shapes and output) every set's a_mx and w_mx, with
// a_mx_rows >= a_rows.
hipError_t launch_tiled_gemm(const GArgs& g, int shape, bool gated, int w_dtype, int out_dtype,
                             int a_dtype, hipStream_t s);
int tiled_bm(int shape);
int tiled_k_multiple();                      // every K (slice) must be a multiple of this
int tiled_k_multiple_a8();                   // the same with fp8 activations
int tiled_k_multiple_small();                // the same for TILED_SMALL
int tiled_blocks_n(int shape, bool gated, int n_out);
// The tiled GEMM addresses A rows and one group's weights with 32-bit byte offsets.
bool tiled_offsets_fit(int64_t a_rows, int64_t lda, int64_t w_rows, int64_t K, int w_dtype);

// Dynamic per-row fp8 quantisation of bf16 rows: scale[r] = max|a[r]| / 448
// (1 for a zero row), q[r][c] = e4m3fn(a[r][c] / scale[r]) rounded to nearest
// even, saturating.  cols % 8 == 0, cols <= quant_max_cols(); q is [rows][cols].
int quant_max_cols();
hipError_t launch_quant_rows(const uint16_t* a, int rows, int cols, int64_t lda, uint8_t* q,
                             float* scale, hipStream_t s);
// The same per kSubChannel-element slice of each row: scale[u * rows + r] for
// slice u.  cols % kSubChannel == 0, cols <= quant_max_cols().
hipError_t launch_quant_rows_sub(const uint16_t* a, int rows, int cols, int64_t lda, uint8_t* q,
                                 float* scale, hipStream_t s);
// MXFP8 quantisation of bf16 rows: per block of 32 elements an E8M0 scale
// 2^(floor(log2 amax) - 8) (clamped to [2^-127, 2^127]; 2^-127 for a zero
// block) and e4m3fn codes of a / scale (nearest even, saturating).  Scales go
// to scale[(c / 128) * rows + r][(c % 128) / 32] (rows side by side per group of
// 128 columns).
// cols % 128 == 0, cols <= quant_max_cols().
hipError_t launch_quant_rows_mx(const uint16_t* a, int rows, int cols, int64_t lda, uint8_t* q,
                                uint8_t* scale, hipStream_t s);

// Decode n (multiple of 8) fp8 e4m3fn codes to bf16 with the GEMM's own decoder.
hipError_t launch_fp8_decode(const uint8_t* codes, uint16_t* out, int n, hipStream_t s);
hipError_t launch_fp8_encode(const float* v, uint8_t* out, int n, hipStream_t s);

// Measurement probes: a streaming read of `bytes` (a multiple of 16) with
// eight 16-byte loads in flight per thread (sink: 1024 words, written only on
// a magic XOR value); independent register-only MFMAs (bf16 16x16x32 or fp8
// 32x32x64) on operands read from 64 KiB of random values, with the FLOP
// count of the launch in *flop (sink: probe_mfma_threads() floats).
int probe_mfma_threads();
hipError_t launch_probe_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t s);
hipError_t launch_probe_mfma(bool fp8, const void* operands, int iters, float* sink, double* flop,
                             hipStream_t s);

// Combine.
// Sets n int32 values to v (a kernel, so it can be captured in a graph).
hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s);

hipError_t launch_combine(const void* o_perm, const int32_t* row_of_slot, const float* w,
                          const void* shared, int T, int D, int k, int dtype, void* y,
                          hipStream_t s);

}  // namespace moe
