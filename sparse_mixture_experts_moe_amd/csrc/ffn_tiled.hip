// LDS-tiled grouped GEMM for large groups (prefill-sized batches).
//
// Prefill is bound by the MFMA units once every expert has hundreds of rows
// ("Qwen 3.5 MoE on Ironwood", roofline section: prefill is compute-bound and
// uneven expert loads make padding in the grouped GEMM the thing to minimise;
// "Ling-2.6-1T with SGLang-JAX", section 4: keep tokens and accumulators
// resident and double-buffer the expert weights).  Each block owns one M-tile
// of a group (up to 128 sorted rows, so a group is padded to a multiple of 128
// rows at most) and 256 weight rows; the K dimension is staged through LDS 64
// elements at a time with two buffers, so the global loads of stage s+1 are in
// flight while the MFMAs of stage s run.
//
// Block: 256 threads = 4 wavefronts in a 2 x 2 grid, each computing a 64-row x
// 128-column slab with 16x16x32 bf16 MFMAs (4 x 8 accumulator tiles).  For the
// fused gate/up projection the 256 weight rows are 128 gate rows followed by
// the 128 matching up rows; a wavefront's columns are 64 gate + 64 up of the
// same h columns, so act(gate)*up is formed in registers and only h is written.
//
// LDS rows are 64 bf16 = 128 bytes = 8 chunks of 16 bytes; chunk c of row r is
// stored at chunk position c ^ (r & 7), which keeps both the 16-byte stores of
// the global->LDS copy and the 16-byte fragment reads free of bank conflicts.
// fp8 e4m3fn weights are decoded exactly to bf16 on the way into LDS and their
// per-channel scales are applied after the reduction.
#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int BM = 128;                    // rows per M-tile
constexpr int BNW = 256;                   // weight rows per block
constexpr int BK = 64;                     // K elements per stage
constexpr int THREADS = 256;
constexpr int ROWB = BK * 2;               // LDS bytes per tile row
constexpr int A_BYTES = BM * ROWB;         // 16 KiB
constexpr int B_BYTES = BNW * ROWB;        // 32 KiB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * ROWB + ((chunk ^ (row & 7)) << 4);
}

template <bool GATED, int WDT, int ODT>
__global__ __launch_bounds__(THREADS, 1) void tiled_gemm_kernel(const GArgs g) {
  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE_BYTES];
  int si, group, row0, row1, nblk;
  if (!resolve_block(g, blockIdx.x, si, group, row0, row1, nblk)) return;
  const GSet& S = g.s[si];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int K = S.K;
  // K slice of this block (plain fp32 outputs may be split into partial sums)
  const int split = S.ksplit > 1 ? static_cast<int>((blockIdx.x - S.block0) % S.ksplit) : 0;
  const int k_len = S.ksplit > 1 ? K / S.ksplit : K;
  const int k_beg = split * k_len;
  const int nst = k_len / BK;
  const int n_out = S.n_out;
  const int n0 = nblk * (GATED ? BNW / 2 : BNW);   // first h column (gated) / output column

  // ---- global -> LDS copy assignments
  // A: 128 rows x 8 chunks; thread covers chunk tid%8 of rows tid/8 + 32 i
  const int ac = tid & 7;
  const char* a_ptr[4];
  bool a_ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = row0 + (tid >> 3) + 32 * i;
    a_ok[i] = r < row1;
    int64_t arow = 0;
    if (a_ok[i]) {
      arow = S.gather ? S.gather[r] : r;
      if (static_cast<uint64_t>(arow) >= static_cast<uint64_t>(S.a_rows)) {
        a_ok[i] = false;
        arow = 0;
      }
    }
    a_ptr[i] = static_cast<const char*>(S.a) + (arow * S.lda + k_beg + ac * 8) * 2;
  }
  // B: tile row tr -> weight row; bf16: 8 chunks of 8 rows per thread, fp8: 4 x 16 bytes
  constexpr int BL = WDT == DT_FP8 ? 4 : 8;         // 16-byte loads per thread per stage
  constexpr int BSTEP = WDT == DT_FP8 ? 64 : 32;    // tile-row step between a thread's loads
  const int bc = WDT == DT_FP8 ? (tid & 3) : (tid & 7);
  const int brow0 = WDT == DT_FP8 ? (tid >> 2) : (tid >> 3);
  const char* wg = static_cast<const char*>(S.w) + group * S.w_gstride * (WDT == DT_FP8 ? 1 : 2);
  const char* b_ptr[BL];
  bool b_ok[BL];
#pragma unroll
  for (int i = 0; i < BL; ++i) {
    const int tr = brow0 + BSTEP * i;
    int wrow;
    if (GATED) {
      const int n = n0 + (tr & (BNW / 2 - 1));
      b_ok[i] = n < n_out;
      wrow = (tr < BNW / 2 ? 0 : n_out) + n;
    } else {
      wrow = n0 + tr;
      b_ok[i] = wrow < n_out;
    }
    if (!b_ok[i]) wrow = 0;
    if constexpr (WDT == DT_FP8)
      b_ptr[i] = wg + static_cast<int64_t>(wrow) * K + k_beg + bc * 16;
    else
      b_ptr[i] = wg + (static_cast<int64_t>(wrow) * K + k_beg + bc * 8) * 2;
  }

  uint4 ra[4], rb[BL];
  auto gload = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ra[i] = a_ok[i] ? *reinterpret_cast<const uint4*>(a_ptr[i] + st * (BK * 2)) : uint4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int64_t off = static_cast<int64_t>(st) * BK * (WDT == DT_FP8 ? 1 : 2);
      rb[i] = b_ok[i] ? *reinterpret_cast<const uint4*>(b_ptr[i] + off) : uint4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
    char* base = smem + buf * STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(base + swz((tid >> 3) + 32 * i, ac)) = ra[i];
    char* bb = base + A_BYTES;
#pragma unroll
    for (int i = 0; i < BL; ++i) {
      const int tr = brow0 + BSTEP * i;
      if constexpr (WDT == DT_FP8) {
        const bf16x8 lo = fp8x8_to_bf16x8(rb[i].x, rb[i].y);
        const bf16x8 hi = fp8x8_to_bf16x8(rb[i].z, rb[i].w);
        *reinterpret_cast<bf16x8*>(bb + swz(tr, 2 * bc)) = lo;
        *reinterpret_cast<bf16x8*>(bb + swz(tr, 2 * bc + 1)) = hi;
      } else {
        *reinterpret_cast<uint4*>(bb + swz(tr, bc)) = rb[i];
      }
    }
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int f = 0; f < 8; ++f) acc[i][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int lr = lane & 15, q = lane >> 4;
  auto compute = [&](int buf) {
    const char* base = smem + buf * STAGE_BYTES;
    const char* bb = base + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      const int chunk = ks * 4 + q;
      bf16x8 af[4], bfr[8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(base + swz(wm * 64 + i * 16 + lr, chunk));
#pragma unroll
      for (int f = 0; f < 8; ++f) {
        const int tr = GATED ? ((f < 4 ? 0 : BNW / 2) + wn * 64 + (f & 3) * 16 + lr)
                             : (wn * 128 + f * 16 + lr);
        bfr[f] = *reinterpret_cast<const bf16x8*>(bb + swz(tr, chunk));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int f = 0; f < 8; ++f)
          acc[i][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[f], acc[i][f], 0, 0, 0);
    }
  };

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

  // ---- epilogue: fragment (i, f) holds C[row 4q + j][col lr]
  const float* sc = S.scale ? S.scale + group * S.s_gstride : nullptr;
  char* out = static_cast<char*>(S.out) + split * S.split_stride * (ODT == DT_F32 ? 4 : 2);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = row0 + wm * 64 + i * 16 + q * 4 + j;
      if (r >= row1) continue;
      if constexpr (GATED) {
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const int col = n0 + wn * 64 + f * 16 + lr;
          if (col >= n_out) continue;
          float gv = acc[i][f][j], uv = acc[i][f + 4][j];
          if (sc) {
            gv *= sc[col];
            uv *= sc[n_out + col];
          }
          const float h = act_fn(S.act, gv) * uv;
          const int64_t o = static_cast<int64_t>(r) * S.ldo + col;
          if constexpr (ODT == DT_F32) reinterpret_cast<float*>(out)[o] = h;
          else reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16(h);
        }
      } else {
#pragma unroll
        for (int f = 0; f < 8; ++f) {
          const int col = n0 + wn * 128 + f * 16 + lr;
          if (col >= n_out) continue;
          float v = acc[i][f][j];
          if (sc) v *= sc[col];
          const int64_t o = static_cast<int64_t>(r) * S.ldo + col;
          if constexpr (ODT == DT_F32) reinterpret_cast<float*>(out)[o] = v;
          else reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16(v);
        }
      }
    }
  }
}

template <bool GATED, int WDT, int ODT>
hipError_t launch_one(const GArgs& g, hipStream_t s) {
  tiled_gemm_kernel<GATED, WDT, ODT><<<g.total_blocks, THREADS, 0, s>>>(g);
  return hipGetLastError();
}

}  // namespace

int tiled_bm() { return BM; }
int tiled_blocks_n(bool gated, int n_out) {
  return gated ? (n_out + BNW / 2 - 1) / (BNW / 2) : (n_out + BNW - 1) / BNW;
}

hipError_t launch_tiled_gemm(const GArgs& g, bool gated, int w_dtype, int out_dtype, hipStream_t s) {
  if (g.total_blocks <= 0) return hipSuccess;
  if (gated) {
    if (w_dtype == DT_BF16 && out_dtype == DT_BF16) return launch_one<true, DT_BF16, DT_BF16>(g, s);
    if (w_dtype == DT_FP8 && out_dtype == DT_BF16) return launch_one<true, DT_FP8, DT_BF16>(g, s);
  } else {
    if (w_dtype == DT_BF16 && out_dtype == DT_BF16) return launch_one<false, DT_BF16, DT_BF16>(g, s);
    if (w_dtype == DT_FP8 && out_dtype == DT_BF16) return launch_one<false, DT_FP8, DT_BF16>(g, s);
    if (w_dtype == DT_BF16 && out_dtype == DT_F32) return launch_one<false, DT_BF16, DT_F32>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
