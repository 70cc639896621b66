// LDS-tiled grouped GEMM for large groups (prefill-sized batches).
//
// Prefill is bound by the MFMA units once every expert has hundreds of rows
// ("Qwen 3.5 MoE on Ironwood", roofline section: prefill is compute-bound and
// uneven expert loads make padding in the grouped GEMM the thing to minimise;
// "Ling-2.6-1T with SGLang-JAX", section 4: keep tokens and accumulators
// resident and stream the expert weights with the next tile's fetch in flight).
//
// Block tile: 128 sorted rows of one group x 256 weight rows; K is staged 32
// elements at a time through two LDS buffers (48 KiB), and the global loads of
// stage s+1 are in flight while the MFMAs of stage s run.  The block is small
// enough in registers (128 accumulators per lane) and LDS for two blocks to be
// resident on a CU, so one block's MFMAs cover the other's barrier and LDS
// waits.  4 wavefronts in a 2 x 2 grid each own 64 rows x 128 weight rows and
// issue 16x16x32 bf16 MFMAs with the weight fragment as the M operand, so a
// lane's accumulator holds 4 consecutive output columns of one row.  For the
// fused gate/up projection the 256 weight rows are 128 gate rows and the 128
// matching up rows; a wavefront holds the gate and up halves of the same 64 h
// columns and forms act(gate)*up in registers (the packed gate/up tile of GMM
// v2 on the Ironwood page).
//
// LDS rows hold 32 bf16 (64 bytes, 4 chunks of 16); chunk c of row r sits at
// c ^ ((r >> 1) & 3), which keeps the 16-byte copy stores and fragment reads
// free of bank conflicts.  fp8 e4m3fn weights stay fp8 in LDS (32-byte rows of
// four 8-byte chunks, chunk c of row r at c ^ ((r >> 2) & 3)) and are decoded
// exactly to bf16 as fragments are read, which halves the weight tile's LDS
// traffic; per-channel scales are applied after the reduction.
//
// Blocks are remapped so that consecutive tiles (the M-tiles and N-blocks of
// one expert) run on the same XCD and share its L2; the remap spans only the
// tiles that exist, so empty tile slots of the grid cost nothing.
#include "moe_kernels.h"

namespace moe {
namespace {

// Build-time tuning knob: MOE_TILED_REMAP 1 = XCD-aware block order.
#ifndef MOE_TILED_REMAP
#define MOE_TILED_REMAP 0
#endif

constexpr int BNW = 256;                  // weight rows per block
constexpr int BK = 32;                    // K elements per stage
constexpr int NSTAGE = 2;                 // LDS buffers
constexpr int THREADS = 256;
constexpr int ROWB = BK * 2;              // LDS bytes per bf16 tile row (64)
constexpr int ROWB8 = BK;                 // LDS bytes per fp8 tile row (32)
constexpr int NXCD = 8;

template <int BM, bool FP8> struct Cfg {
  static constexpr int A_BYTES = BM * ROWB;
  static constexpr int B_BYTES = BNW * (FP8 ? ROWB8 : ROWB);
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int WM = BM / 2;           // rows per wavefront
  static constexpr int TF = WM / 16;          // row (token) fragments per wavefront
  static constexpr int AL = BM / 64;          // A chunks per thread per stage
  static constexpr int LDS = NSTAGE * STAGE;
};

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * ROWB + ((chunk ^ ((row >> 1) & 3)) << 4);
}
__device__ __forceinline__ int swz8(int row, int chunk) {
  return row * ROWB8 + ((chunk ^ ((row >> 2) & 3)) << 3);
}

#if MOE_TILED_REMAP
// Logical tile of a physical block: consecutive logical tiles share an XCD.
__device__ __forceinline__ bool remap_block(const GArgs& g, int& logical) {
  int real = 0;
  for (int i = 0; i < g.nsets; ++i) {
    const GSet& S = g.s[i];
    const int m = S.tiles ? min(S.n_tiles[0], S.m_slots) : S.m_slots;
    real += m * S.blocks_per_m * (S.ksplit > 1 ? S.ksplit : 1);
  }
  const int per_xcd = (real + NXCD - 1) / NXCD;
  const int b = blockIdx.x;
  const int slot = b / NXCD;
  if (slot >= per_xcd) return false;
  logical = (b % NXCD) * per_xcd + slot;
  if (logical >= real) return false;
  // turn the dense logical index back into the grid numbering resolve_block uses
  int acc = 0;
  for (int i = 0; i < g.nsets; ++i) {
    const GSet& S = g.s[i];
    const int m = S.tiles ? min(S.n_tiles[0], S.m_slots) : S.m_slots;
    const int n = m * S.blocks_per_m * (S.ksplit > 1 ? S.ksplit : 1);
    if (logical < acc + n) {
      logical = S.block0 + (logical - acc);
      return true;
    }
    acc += n;
  }
  return false;
}
#endif

template <int BM, bool GATED, int WDT, int ODT>
__global__ __launch_bounds__(THREADS, 2) void tiled_gemm_kernel(const GArgs g) {
  using C = Cfg<BM, WDT == DT_FP8>;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS];
  // An (empty) statement that names an accumulation register makes the backend
  // select the AGPR form of the MFMAs, so the accumulators live in AGPRs and
  // the VGPRs stay free for fragments and the copy pipeline.
  asm volatile("" ::: "a0");
  int b = blockIdx.x;
#if MOE_TILED_REMAP
  if (!remap_block(g, b)) return;
#endif
  int si, group, row0, row1, nblk;
  if (!resolve_block(g, b, si, group, row0, row1, nblk)) return;
  const GSet& S = g.s[si];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int lr = lane & 15, q = lane >> 4;
  const int K = S.K;
  const int split = S.ksplit > 1 ? (b - S.block0) % S.ksplit : 0;
  const int k_len = S.ksplit > 1 ? K / S.ksplit : K;
  const int k_beg = split * k_len;
  const int nst = k_len / BK;
  const int n_out = S.n_out;
  const int n0 = nblk * (GATED ? BNW / 2 : BNW);   // first h column (gated) / output column

  // ---- global -> LDS copy assignments (A: BM rows x 4 chunks, thread: chunk tid%4).
  // Rows past the tile and weight rows past n_out are loaded from a valid row
  // instead: they only feed accumulator rows / columns the epilogue never stores,
  // so the copy needs no per-load predication.
  const int cc = tid & 3;
  const char* a_ptr[C::AL];
#pragma unroll
  for (int i = 0; i < C::AL; ++i) {
    const int r = row0 + (tid >> 2) + 64 * i;
    int64_t arow = 0;
    if (r < row1) {
      arow = S.gather ? S.gather[r] : r;
      if (static_cast<uint64_t>(arow) >= static_cast<uint64_t>(S.a_rows)) arow = 0;  // caller error
    }
    a_ptr[i] = static_cast<const char*>(S.a) + (arow * S.lda + k_beg + cc * 8) * 2;
  }
  // B: bf16 -> 4 rows x 16 B per thread; fp8 -> 2 rows x 16 B (32 codes, 2 LDS chunks each)
  constexpr bool FP8 = WDT == DT_FP8;
  constexpr int BL = FP8 ? 2 : 4;
  constexpr int BSTEP = FP8 ? 128 : 64;
  const int bcol = FP8 ? (tid & 1) : cc;
  const int brow0 = FP8 ? (tid >> 1) : (tid >> 2);
  const char* wg = static_cast<const char*>(S.w) + group * S.w_gstride * (FP8 ? 1 : 2);
  const char* b_ptr[BL];
#pragma unroll
  for (int i = 0; i < BL; ++i) {
    const int tr = brow0 + BSTEP * i;
    int wrow;
    if (GATED) {
      const int n = n0 + (tr & (BNW / 2 - 1));
      wrow = n < n_out ? (tr < BNW / 2 ? 0 : n_out) + n : 0;
    } else {
      wrow = n0 + tr < n_out ? n0 + tr : 0;
    }
    b_ptr[i] = FP8 ? wg + static_cast<int64_t>(wrow) * K + k_beg + bcol * 16
                   : wg + (static_cast<int64_t>(wrow) * K + k_beg + bcol * 8) * 2;
  }

  // one register stage in flight
  u32x4 ra[C::AL], rb[BL];
  auto gload = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::AL; ++i)
      ra[i] = *reinterpret_cast<const u32x4*>(a_ptr[i] + st * (BK * 2));
    const int64_t boff = static_cast<int64_t>(st) * BK * (FP8 ? 1 : 2);
#pragma unroll
    for (int i = 0; i < BL; ++i)
      rb[i] = *reinterpret_cast<const u32x4*>(b_ptr[i] + boff);
  };
  auto lstore = [&](int buf) __attribute__((always_inline)) {
    char* base = smem + buf * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::AL; ++i)
      *reinterpret_cast<u32x4*>(base + swz((tid >> 2) + 64 * i, cc)) = ra[i];
    char* bb = base + C::A_BYTES;
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int tr = brow0 + BSTEP * i;
      if constexpr (FP8) {
        const u32x4 v = rb[i];
        *reinterpret_cast<uint2*>(bb + swz8(tr, 2 * bcol)) = uint2{v[0], v[1]};
        *reinterpret_cast<uint2*>(bb + swz8(tr, 2 * bcol + 1)) = uint2{v[2], v[3]};
      } else {
        *reinterpret_cast<u32x4*>(bb + swz(tr, cc)) = rb[i];
      }
    }
  };

  // acc[f][i]: weight fragment f (16 weight rows) x row fragment i (16 rows)
  f32x4 acc[8][C::TF];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int i = 0; i < C::TF; ++i) acc[f][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf) __attribute__((always_inline)) {
    const char* base = smem + buf * C::STAGE;
    const char* bb = base + C::A_BYTES;
    bf16x8 wf[8], tf[C::TF];
#pragma unroll
    for (int f = 0; f < 8; ++f) {
      const int tr = GATED ? ((f < 4 ? 0 : BNW / 2) + wn * 64 + (f & 3) * 16 + lr)
                           : (wn * 128 + f * 16 + lr);
      if constexpr (WDT == DT_FP8) {
        const uint2 raw = *reinterpret_cast<const uint2*>(bb + swz8(tr, q));
        wf[f] = fp8x8_to_bf16x8(raw.x, raw.y);
      } else {
        wf[f] = *reinterpret_cast<const bf16x8*>(bb + swz(tr, q));
      }
    }
#pragma unroll
    for (int i = 0; i < C::TF; ++i)
      tf[i] = *reinterpret_cast<const bf16x8*>(base + swz(wm * C::WM + i * 16 + lr, q));
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
      for (int i = 0; i < C::TF; ++i)
        acc[f][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[f], tf[i], acc[f][i], 0, 0, 0);
  };

  // ---- pipeline: stage s+1 is fetched into registers while stage s is
  // multiplied out of LDS, then stored to the other buffer; one barrier per stage.
  gload(0);
  lstore(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const bool more = st + 1 < nst;
    if (more) gload(st + 1);
    compute(st & 1);
    if (more) lstore((st + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds C[row lr of fragment i][cols 4q..4q+3 of fragment f];
  // the 4 columns are stored together (8 bytes in bf16, 16 in fp32).
  const float* sc = S.scale ? S.scale + group * S.s_gstride : nullptr;
  constexpr int OCOLS = GATED ? 64 : 128;      // output columns per wavefront
  const int col_w = n0 + wn * OCOLS;           // first output column of this wavefront
  char* outb = static_cast<char*>(S.out) + split * S.split_stride * (ODT == DT_F32 ? 4 : 2);
#pragma unroll
  for (int i = 0; i < C::TF; ++i) {
    const int r = row0 + wm * C::WM + i * 16 + lr;
    if (r >= row1) continue;
#pragma unroll
    for (int f = 0; f < (GATED ? 4 : 8); ++f) {
      const int col = col_w + f * 16 + 4 * q;  // first of the lane's 4 columns
      if (col >= n_out) continue;              // n_out is a multiple of 4
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (GATED) {
          float gv = acc[f][i][j], uv = acc[f + 4][i][j];
          if (sc) {
            gv *= sc[col + j];
            uv *= sc[n_out + col + j];
          }
          v[j] = act_fn(S.act, gv) * uv;
        } else {
          v[j] = acc[f][i][j] * (sc ? sc[col + j] : 1.f);
        }
      }
      const int64_t o = static_cast<int64_t>(r) * S.ldo + col;
      if constexpr (ODT == DT_BF16) {
        const uint32_t p0 = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
        const uint32_t p1 = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(outb) + o) = uint2{p0, p1};
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(outb) + o) = float4{v[0], v[1], v[2], v[3]};
      }
    }
  }
}

template <int BM, bool GATED, int WDT, int ODT>
hipError_t launch_one(const GArgs& g, hipStream_t s) {
  const int grid = MOE_TILED_REMAP ? (g.total_blocks + NXCD - 1) / NXCD * NXCD : g.total_blocks;
  tiled_gemm_kernel<BM, GATED, WDT, ODT><<<grid, THREADS, 0, s>>>(g);
  return hipGetLastError();
}

template <int BM>
hipError_t dispatch(const GArgs& g, bool gated, int w_dtype, int out_dtype, hipStream_t s) {
  if (gated) {
    if (w_dtype == DT_BF16 && out_dtype == DT_BF16) return launch_one<BM, true, DT_BF16, DT_BF16>(g, s);
    if (w_dtype == DT_FP8 && out_dtype == DT_BF16) return launch_one<BM, true, DT_FP8, DT_BF16>(g, s);
  } else {
    if (w_dtype == DT_BF16 && out_dtype == DT_BF16) return launch_one<BM, false, DT_BF16, DT_BF16>(g, s);
    if (w_dtype == DT_FP8 && out_dtype == DT_BF16) return launch_one<BM, false, DT_FP8, DT_BF16>(g, s);
    if (w_dtype == DT_BF16 && out_dtype == DT_F32) return launch_one<BM, false, DT_BF16, DT_F32>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

int tiled_blocks_n(bool gated, int n_out) {
  return gated ? (n_out + BNW / 2 - 1) / (BNW / 2) : (n_out + BNW - 1) / BNW;
}

hipError_t launch_tiled_gemm(const GArgs& g, int bm, bool gated, int w_dtype, int out_dtype,
                             hipStream_t s) {
  if (g.total_blocks <= 0) return hipSuccess;
  for (int i = 0; i < g.nsets; ++i) {
    const int ks = g.s[i].ksplit > 1 ? g.s[i].ksplit : 1;
    if ((g.s[i].K / ks) % BK || g.s[i].bm != bm || g.s[i].n_out % 4) return hipErrorInvalidValue;
  }
  if (bm == 128) return dispatch<128>(g, gated, w_dtype, out_dtype, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
