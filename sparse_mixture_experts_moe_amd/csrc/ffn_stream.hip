// Grouped expert GEMM with weights streamed from HBM straight into registers.
//
// Built for groups of few rows (decode-sized batches), where the expert FFN is
// bound by reading every touched expert's weights once ("Qwen 3.5 MoE on
// Ironwood", roofline section: decode is HBM-bound at about 1 FLOP/byte; the
// "Ling-2.6-1T with SGLang-JAX" page, section 1, HBM weight-movement bound).
// The automatic tile policy runs most decode batches on the LDS-tiled
// kernel's 32-row shape instead, which keeps more weight bytes in flight; this
// kernel serves the fp32 layer, the decode router, sizes that shape does not
// take and the MOE_TILE_STREAM policy.
//
// Work decomposition: each 64-wide wavefront owns one M-tile of a group (up to
// 16*MT sorted rows) and 64 weight rows (4 MFMA fragments of 16).  For the
// fused gate/up projection those are 32 gate rows and the 32 matching up rows,
// so SiLU(gate)*up (or tanh-GELU) is applied in registers and only h is stored
// -- the packed gate/up tile of GMM v2 on the Ironwood page (MoE track), without
// an HBM round trip for the two halves.  Every weight element is loaded by
// exactly one wavefront per M-tile; the activation rows are gathered through
// the permutation (the SparseCore gather of the Ironwood page, fused into the
// A-operand load instead of a materialised permuted copy).
//
// The K loop is software-pipelined over two register stages of 32*U elements.
// In MFMA step u of a stage, lane group q = lane/16 supplies K elements
// [32u + 8q, 32u + 8q + 8) (bf16 / fp32 weights) or, for fp8 weights whose
// 16-byte loads cover two steps, [64(u/2) + 16q + 8(u%2), +8).  Either way the
// four lane groups of one 16-byte load instruction read 64 contiguous bytes of
// each weight row, and A and B use the same K assignment, so each MFMA still
// contracts matching elements.
//
// fp8 e4m3fn weights are decoded exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8,
// scale 1) and their per-output-channel fp32 scale is applied after the
// reduction ("Ling-2.6-1T with SGLang-JAX", section 5, per-channel scaling).
// fp32 problems use fp32 MFMA (16x16x4), never a reduced precision.
#include "moe_kernels.h"

namespace moe {
namespace {

// 16-row weight fragments per wavefront; a gated wavefront holds NF/2 gate
// and NF/2 up fragments
constexpr int NF = 4;
constexpr int WROWS = 16 * NF;   // weight rows per wavefront
constexpr int WAVES = 4;         // wavefronts per block (consecutive N tiles)

__device__ __forceinline__ uint4 load_w(const uint4* p) { return *p; }

template <int DT> struct Elt;
template <> struct Elt<DT_F32> { static constexpr int bytes = 4; };
template <> struct Elt<DT_BF16> { static constexpr int bytes = 2; };
template <> struct Elt<DT_FP8> { static constexpr int bytes = 1; };

// uint4 vectors holding 8*U elements of dtype DT
template <int DT, int U> struct VecCount {
  static constexpr int n = (8 * U * Elt<DT>::bytes) / 16;
};

template <int MT, int U, bool GATED, int ADT, int WDT, int ODT>
__global__ __launch_bounds__(64 * WAVES, 2) void stream_gemm_kernel(const GArgs g) {
  constexpr int AV = VecCount<ADT, U>::n;   // uint4 per lane per stage, A
  constexpr int BV = VecCount<WDT, U>::n;   // uint4 per lane per stage, B (per fragment)
  constexpr int KS = 32 * U;                // K elements per stage
  int si, group, row0, row1, nblk;
  if (!resolve_block(g, blockIdx.x, si, group, row0, row1, nblk)) return;
  const GSet& S = g.s[si];
  const int lane = threadIdx.x & 63;
  const int q = lane >> 4, lr = lane & 15;
  const int wn = nblk * WAVES + (threadIdx.x >> 6);
  const int n_out = S.n_out;
  const int waves_n = GATED ? n_out / (WROWS / 2) : (n_out + WROWS - 1) / WROWS;
  if (wn >= waves_n) return;
  const int K = S.K;
  const int nch = (row1 - row0 + 15) >> 4;  // active 16-row chunks (<= MT)
  // K slice of this block (plain fp32 outputs may be split into partial sums)
  const int split = S.ksplit > 1 ? static_cast<int>((blockIdx.x - S.block0) % S.ksplit) : 0;
  const int k_len = S.ksplit > 1 ? K / S.ksplit : K;
  const int k_beg = split * k_len;

  // ---- operand pointers (element offsets are per lane: row + q*8U)
  const char* a_base = static_cast<const char*>(S.a);
  const char* ap[MT];
  bool av[MT];
#pragma unroll
  for (int mc = 0; mc < MT; ++mc) {
    const int r = row0 + mc * 16 + lr;
    av[mc] = mc < nch && r < row1;
    int64_t arow = 0;
    if (av[mc]) {
      arow = S.gather ? S.gather[r] : r;
      if (static_cast<uint64_t>(arow) >= static_cast<uint64_t>(S.a_rows)) {  // caller error
        av[mc] = false;
        arow = 0;
      }
    }
    ap[mc] = a_base + (arow * S.lda + k_beg) * Elt<ADT>::bytes;
  }
  const char* w_base = static_cast<const char*>(S.w) + group * S.w_gstride * Elt<WDT>::bytes;
  const char* bp[NF];
  bool bv[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    int n;
    if (GATED) {
      n = (f < NF / 2 ? 0 : n_out) + wn * (WROWS / 2) + (f % (NF / 2)) * 16 + lr;
      bv[f] = true;
    } else {
      n = wn * WROWS + f * 16 + lr;
      bv[f] = n < n_out;
      if (!bv[f]) n = 0;
    }
    bp[f] = w_base + (static_cast<int64_t>(n) * K + k_beg) * Elt<WDT>::bytes;
  }

  f32x4 acc[MT][NF];
#pragma unroll
  for (int mc = 0; mc < MT; ++mc)
#pragma unroll
    for (int f = 0; f < NF; ++f) acc[mc][f] = f32x4{0.f, 0.f, 0.f, 0.f};

  uint4 sa0[MT][AV], sb0[NF][BV], sa1[MT][AV], sb1[NF][BV];

  // byte offset of 16-byte vector v of a stage, for operand dtype DT, in the K
  // assignment described at the top of the file
  auto voff = [&](int dt_bytes, int v) __attribute__((always_inline)) -> int {
    if (dt_bytes == 1) return v * 64 + q * 16;                         // fp8 weights: pairs of steps
    if (dt_bytes == 4) return (v >> 1) * 128 + q * 32 + (v & 1) * 16;  // fp32: two vectors per step
    if (WDT == DT_FP8) return (v >> 1) * 128 + q * 32 + (v & 1) * 16;  // bf16 A beside fp8 weights
    return v * 64 + q * 16;                                            // bf16, one vector per step
  };
  auto load = [&](uint4 (&sa)[MT][AV], uint4 (&sb)[NF][BV], int stage) __attribute__((always_inline)) {
    const int64_t koff = static_cast<int64_t>(stage) * KS;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const char* p = bp[f] + koff * Elt<WDT>::bytes;
#pragma unroll
      for (int v = 0; v < BV; ++v)
        sb[f][v] = bv[f] ? load_w(reinterpret_cast<const uint4*>(p + voff(Elt<WDT>::bytes, v)))
                         : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int mc = 0; mc < MT; ++mc) {
      const char* p = ap[mc] + koff * Elt<ADT>::bytes;
#pragma unroll
      for (int v = 0; v < AV; ++v)
        sa[mc][v] = av[mc] ? *reinterpret_cast<const uint4*>(p + voff(Elt<ADT>::bytes, v))
                           : uint4{0, 0, 0, 0};
    }
  };

  auto compute = [&](const uint4 (&sa)[MT][AV], const uint4 (&sb)[NF][BV]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if constexpr (ADT == DT_F32) {
        // fp32: eight 16x16x4 MFMAs per 8 K-elements; element i of every lane
        // group forms the K=4 slice of the i-th instruction.
#pragma unroll
        for (int mc = 0; mc < MT; ++mc) {
          if (mc < nch) {
            const float* af = reinterpret_cast<const float*>(&sa[mc][2 * u]);
#pragma unroll
            for (int f = 0; f < NF; ++f) {
              const float* bf = reinterpret_cast<const float*>(&sb[f][2 * u]);
#pragma unroll
              for (int i = 0; i < 8; ++i)
                acc[mc][f] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bf[i], acc[mc][f], 0, 0, 0);
            }
          }
        }
      } else {
        bf16x8 bo[NF];
#pragma unroll
        for (int f = 0; f < NF; ++f) bo[f] = operand_bf16<WDT>(sb[f], u);
#pragma unroll
        for (int mc = 0; mc < MT; ++mc) {
          if (mc < nch) {
            const bf16x8 ao = __builtin_bit_cast(bf16x8, sa[mc][u]);
#pragma unroll
            for (int f = 0; f < NF; ++f)
              acc[mc][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ao, bo[f], acc[mc][f], 0, 0, 0);
          }
        }
      }
    }
  };

  const int nst = k_len / KS;
  load(sa0, sb0, 0);
  for (int st = 0; st < nst; st += 2) {
    if (st + 1 < nst) load(sa1, sb1, st + 1);
    compute(sa0, sb0);
    if (st + 1 < nst) {
      if (st + 2 < nst) load(sa0, sb0, st + 2);
      compute(sa1, sb1);
    }
  }

  // ---- epilogue: C[row = 4*q + j][col = lr] of each 16x16 fragment
  const float* sc = S.scale ? S.scale + group * S.s_gstride : nullptr;
  char* out = static_cast<char*>(S.out) + split * S.split_stride * Elt<ODT>::bytes;
#pragma unroll
  for (int mc = 0; mc < MT; ++mc) {
    if (mc >= nch) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = row0 + mc * 16 + q * 4 + j;
      if (r >= row1) continue;
      if constexpr (GATED) {
#pragma unroll
        for (int f = 0; f < NF / 2; ++f) {
          const int col = wn * (WROWS / 2) + f * 16 + lr;
          float gv = acc[mc][f][j], uv = acc[mc][f + NF / 2][j];
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
        for (int f = 0; f < NF; ++f) {
          const int col = wn * WROWS + f * 16 + lr;
          if (col >= n_out) continue;
          float v = acc[mc][f][j];
          if (sc) v *= sc[col];
          const int64_t o = static_cast<int64_t>(r) * S.ldo + col;
          if constexpr (ODT == DT_F32) reinterpret_cast<float*>(out)[o] = v;
          else reinterpret_cast<uint16_t*>(out)[o] = f32_to_bf16(v);
        }
      }
    }
  }
}

template <int MT, int U, bool GATED, int ADT, int WDT, int ODT>
hipError_t launch_one(const GArgs& g, hipStream_t s) {
  stream_gemm_kernel<MT, U, GATED, ADT, WDT, ODT><<<g.total_blocks, 64 * WAVES, 0, s>>>(g);
  return hipGetLastError();
}

template <int MT, bool GATED, int ADT, int WDT, int ODT>
hipError_t pick_u(const GArgs& g, hipStream_t s) {
  // K-steps per register stage (measured): four for two-chunk tiles of
  // bf16/fp8 operands when every K allows, two otherwise (one- and four-chunk
  // tiles, fp32 operands)
  if constexpr (MT == 2 && ADT != DT_F32) {
    bool k128 = true;
    for (int i = 0; i < g.nsets; ++i)
      k128 = k128 && (g.s[i].K / (g.s[i].ksplit > 1 ? g.s[i].ksplit : 1)) % 128 == 0;
    if (k128) return launch_one<MT, 4, GATED, ADT, WDT, ODT>(g, s);
  }
  return launch_one<MT, 2, GATED, ADT, WDT, ODT>(g, s);
}

template <bool GATED, int ADT, int WDT, int ODT>
hipError_t pick_mt(const GArgs& g, int mt, hipStream_t s) {
  if (mt == 1) return pick_u<1, GATED, ADT, WDT, ODT>(g, s);
  if constexpr (ADT == DT_F32) {
    return pick_u<2, GATED, ADT, WDT, ODT>(g, s);  // fp32: at most 32-row tiles
  } else {
    if (mt == 2) return pick_u<2, GATED, ADT, WDT, ODT>(g, s);
    return pick_u<4, GATED, ADT, WDT, ODT>(g, s);
  }
}

template <bool GATED>
hipError_t pick_types(const GArgs& g, int mt, int a_dt, int w_dt, int o_dt, hipStream_t s) {
  if (a_dt == DT_F32 && w_dt == DT_F32 && o_dt == DT_F32)
    return pick_mt<GATED, DT_F32, DT_F32, DT_F32>(g, mt, s);
  if (a_dt == DT_BF16 && w_dt == DT_BF16 && o_dt == DT_BF16)
    return pick_mt<GATED, DT_BF16, DT_BF16, DT_BF16>(g, mt, s);
  if (a_dt == DT_BF16 && w_dt == DT_FP8 && o_dt == DT_BF16)
    return pick_mt<GATED, DT_BF16, DT_FP8, DT_BF16>(g, mt, s);
  if (!GATED && a_dt == DT_BF16 && w_dt == DT_BF16 && o_dt == DT_F32)
    return pick_mt<GATED, DT_BF16, DT_BF16, DT_F32>(g, mt, s);
  return hipErrorInvalidValue;
}

__global__ void fp8_decode_kernel(const uint8_t* __restrict__ codes, uint16_t* __restrict__ out,
                                  int n) {
  const int i = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i >= n) return;
  const uint2 q = *reinterpret_cast<const uint2*>(codes + i);
  const bf16x8 v = fp8x8_to_bf16x8(q.x, q.y);
  *reinterpret_cast<bf16x8*>(out + i) = v;
}

}  // namespace

hipError_t launch_fp8_decode(const uint8_t* codes, uint16_t* out, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  fp8_decode_kernel<<<(n / 8 + 255) / 256, 256, 0, s>>>(codes, out, n);
  return hipGetLastError();
}

int stream_waves_n(bool gated, int n_out) {
  return gated ? n_out / (WROWS / 2) : (n_out + WROWS - 1) / WROWS;
}

int stream_max_mt(int a_dtype) { return a_dtype == DT_F32 ? 2 : 4; }

hipError_t launch_stream_gemm(const GArgs& g, int mt, bool gated, int a_dtype, int w_dtype,
                              int out_dtype, hipStream_t s) {
  if (g.total_blocks <= 0) return hipSuccess;
  return gated ? pick_types<true>(g, mt, a_dtype, w_dtype, out_dtype, s)
               : pick_types<false>(g, mt, a_dtype, w_dtype, out_dtype, s);
}

}  // namespace moe
