// Internal declarations shared by the HIP sources of the MoE library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ------------------------------------------------------------------ dtypes
enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2 };
enum : int { ACT_SILU = 0, ACT_GELU_TANH = 1 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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
  const void* w;            // [groups][NB][K] weight storage
  const float* scale;       // [groups][NB] per-output-channel scales or null
  int64_t w_gstride;        // elements between groups (NB*K)
  int64_t s_gstride;        // scale elements between groups (NB)
  int32_t NB;               // weight rows: 2*I (gated) or N (plain)
  int32_t n_out;            // output columns: I (gated) or N (plain)
  int32_t act;              // gated activation
  int32_t pad0;
  void* out;                // output storage, row stride ldo elements
  int64_t ldo;
  const GTile* tiles;       // m-tile table, or null for dense tiles over [0, rows)
  const int32_t* n_tiles;   // device count of valid table entries
  int32_t rows;             // dense: number of rows
  int32_t m_slots;          // m-tile slots the grid reserves for this set
  int32_t block0;           // first block id of this set
  int32_t blocks_per_m;     // blocks per m-tile slot (N direction)
  int32_t bm;               // rows per m-tile
  int32_t pad1;
};

struct GArgs {
  GSet s[2];
  int32_t nsets;
  int32_t total_blocks;
};

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error.

// logits[T,E] (fp32) -> topk idx / weights.
hipError_t launch_topk_softmax(const float* logits, int T, int E, int k, int32_t* idx,
                               float* w, hipStream_t s);

// Permutation: per-block bit masks -> counts/offsets -> stable scatter.
int perm_blocks(int T);
hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* blk /*[nb*E]*/,
                          int32_t* local_rank /*[T*k]*/, int32_t* counts, int32_t* offsets,
                          int32_t* row_token, int32_t* row_of_slot, hipStream_t s);

// M-tile table of n_groups groups from device offsets (largest group first).
// Offsets are clamped to [0, max_rows] and at most max_tiles entries are written.
hipError_t launch_build_tiles(const int32_t* offsets, int n_groups, int bm, int max_rows,
                              int max_tiles, GTile* tiles, int32_t* n_tiles, hipStream_t s);

// Grouped GEMM, streamed weights.  mt = 16-row chunks per m-tile (1, 2, 4).
// gated: h = act(A.Wg^T * sg) * (A.Wu^T * su); plain: out = A.W^T * s.
// a_dtype / w_dtype / out_dtype: DT_*.
hipError_t launch_stream_gemm(const GArgs& g, int mt, bool gated, int a_dtype, int w_dtype,
                              int out_dtype, hipStream_t s);
int stream_waves_n(bool gated, int n_out);   // wave tiles along N per m-tile
int stream_max_mt(int a_dtype);              // largest mt the stream kernel runs for a dtype

// Grouped GEMM, LDS-tiled (bf16 activations, bf16 or fp8 weights).
hipError_t launch_tiled_gemm(const GArgs& g, bool gated, int w_dtype, int out_dtype,
                             hipStream_t s);
int tiled_bm();
int tiled_blocks_n(bool gated, int n_out);

// Decode n (multiple of 8) fp8 e4m3fn codes to bf16 with the GEMM's own decoder.
hipError_t launch_fp8_decode(const uint8_t* codes, uint16_t* out, int n, hipStream_t s);

// Combine.
hipError_t launch_combine(const void* o_perm, const int32_t* row_of_slot, const float* w,
                          const void* shared, int T, int D, int k, int dtype, void* y,
                          hipStream_t s);

}  // namespace moe
