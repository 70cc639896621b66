// Dynamic per-row fp8 e4m3fn quantisation of bf16 activation rows: the
// activation quantisation of the "Ling-2.6-1T with SGLang-JAX" page, section
// 5 (tokens quantised from bf16 to fp8 per token, dynamically, before they go
// into the matrix unit with the fp8 weights).
//
// A row's 16-byte chunks stay in registers between the max pass and the
// conversion pass, so a row is read from HBM once.  The scale
// is max|a| / 448 (448 being the largest finite e4m3fn magnitude; 1 for a row
// of zeros), each element becomes the e4m3fn code nearest to a / scale (ties
// to the even code, saturating at +-448), with both divisions correctly
// rounded in fp32.
//
// The sub-channel variant (the GMM v2 kernel of the "Qwen 3.5 MoE on
// Ironwood" page, MoE track: fp8 activations with one scale per 512-element
// sub-channel) applies the same rule to each 512-element slice of a row; a
// wavefront's register chunk u (64 lanes x 8 elements) is exactly slice u,
// so each slice's max is one butterfly.  Its scales are stored slice-major,
// [cols / 512][rows], the layout the GEMM's per-stage scale copies read.
//
// The MXFP8 variant is the activation side of the W4A8 decomposition ("CANN
// Qwen3-MoE" page, high-throughput prefill), with the OCP microscaling block
// format: per 32 elements an E8M0 scale 2^(floor(log2 amax) - 8), clamped to
// exponents [-127, 127], and e4m3fn codes of a / scale; the scaling is an
// exact power of two, so only the code rounding (nearest even) is inexact.
#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int QMAX = 16384;           // widest row: 64 lanes x 32 chunks of 8
static_assert(kSubChannel == 64 * 8, "a sub-channel slice is one chunk per lane");

// e4m3fn codes of a pair of values within +-448 (low byte: a), the nearest
// representable value with ties to the even code: the hardware fp32 -> fp8
// pair conversion, which on this target produces the e4m3fn format (bias 7,
// subnormals m * 2^-9, no infinities).  Checked against the format's
// definition by moe_debug_f32_to_fp8 (every fp32 value from 2^-20 to 448,
// both signs, gave the same codes as a bit-level encoder of the format).
__device__ __forceinline__ uint32_t e4m3_pair(float a, float b) {
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// One wavefront per row, 4 rows per block: lane l holds the row's 16-byte
// chunks l, l + 64, ... (NCH of them) in registers between the max and the
// conversion, so a row is read once and the reduction is a wavefront butterfly.
// SUB: one scale per 512-element slice (chunk group u), scale[u * rows + r].
template <int NCH, bool SUB>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ a, int rows,
                                                         int cols, int64_t lda, uint8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const uint16_t* row = a + r * lda;
  const int nch = cols / 8;
  uint4 v[NCH];
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int c = lane + 64 * u;
    v[u] = c < nch ? *reinterpret_cast<const uint4*>(row + 8 * c) : uint4{0, 0, 0, 0};
  }
  float amax[SUB ? NCH : 1];
#pragma unroll
  for (int u = 0; u < (SUB ? NCH : 1); ++u) amax[u] = 0.f;
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    float& m = amax[SUB ? u : 0];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      m = fmaxf(m, fabsf(__uint_as_float(w[j] << 16)));
      m = fmaxf(m, fabsf(__uint_as_float(w[j] & 0xFFFF0000u)));
    }
  }
  float sc[SUB ? NCH : 1];
#pragma unroll
  for (int u = 0; u < (SUB ? NCH : 1); ++u) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax[u] = fmaxf(amax[u], __shfl_xor(amax[u], off, 64));
    sc[u] = amax[u] > 0.f ? __fdiv_rn(amax[u], 448.0f) : 1.0f;
  }
  uint8_t* qrow = q + r * cols;
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int c = lane + 64 * u;
    if (c >= nch) continue;
    const float s = sc[SUB ? u : 0];
    const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
    uint32_t packed[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x0 = __uint_as_float(w[j] << 16), x1 = __uint_as_float(w[j] & 0xFFFF0000u);
      const uint32_t pair = e4m3_pair(clamp448(__fdiv_rn(x0, s)), clamp448(__fdiv_rn(x1, s)));
      packed[j >> 1] |= pair << (16 * (j & 1));
    }
    *reinterpret_cast<uint2*>(qrow + 8 * c) = uint2{packed[0], packed[1]};
  }
  if (lane == 0) {
    if constexpr (SUB) {
#pragma unroll
      for (int u = 0; u < NCH; ++u)
        if (512 * u < cols) scale[static_cast<int64_t>(u) * rows + r] = sc[u];
    } else {
      scale[r] = sc[0];
    }
  }
}

// MXFP8: lane l's chunks l, l + 64, ...; the four chunks of a 32-element block
// sit in four consecutive lanes, so a block's max is a butterfly over them.
template <int NCH>
__global__ __launch_bounds__(256) void quant_rows_mx_kernel(const uint16_t* __restrict__ a, int rows,
                                                            int cols, int64_t lda, uint8_t* __restrict__ q,
                                                            uint8_t* __restrict__ scale) {
  const int64_t r = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const uint16_t* row = a + r * lda;
  const int nch = cols / 8;
  uint8_t* qrow = q + r * cols;
#pragma unroll
  for (int u = 0; u < NCH; ++u) {
    const int c = lane + 64 * u;      // chunk; block c / 4 (uniform validity per block of 4 lanes)
    const uint4 v = c < nch ? *reinterpret_cast<const uint4*>(row + 8 * c) : uint4{0, 0, 0, 0};
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      amax = fmaxf(amax, fabsf(__uint_as_float(w[j] << 16)));
      amax = fmaxf(amax, fabsf(__uint_as_float(w[j] & 0xFFFF0000u)));
    }
    amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
    // shared exponent floor(log2 amax) - 8 (e4m3fn's largest exponent), exact
    int ex = -127;
    if (amax > 0.f) {
      int e2;
      (void)frexpf(amax, &e2);        // amax = m * 2^e2, m in [0.5, 1)
      ex = min(127, max(-127, e2 - 1 - 8));
    }
    if (c >= nch) continue;
    uint32_t packed[2] = {0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float x0 = ldexpf(__uint_as_float(w[j] << 16), -ex);
      const float x1 = ldexpf(__uint_as_float(w[j] & 0xFFFF0000u), -ex);
      const uint32_t pair = e4m3_pair(clamp448(x0), clamp448(x1));
      packed[j >> 1] |= pair << (16 * (j & 1));
    }
    *reinterpret_cast<uint2*>(qrow + 8 * c) = uint2{packed[0], packed[1]};
    if ((lane & 3) == 0) {
      const int blk = c / 4;
      scale[(static_cast<int64_t>(blk / 4) * rows + r) * 4 + (blk % 4)] = static_cast<uint8_t>(ex + 127);
    }
  }
}

template <int NCH>
hipError_t go_mx(const uint16_t* a, int rows, int cols, int64_t lda, uint8_t* q, uint8_t* scale,
                 hipStream_t s) {
  quant_rows_mx_kernel<NCH><<<(rows + 3) / 4, 256, 0, s>>>(a, rows, cols, lda, q, scale);
  return hipGetLastError();
}

template <int NCH, bool SUB = false>
hipError_t go(const uint16_t* a, int rows, int cols, int64_t lda, uint8_t* q, float* scale,
              hipStream_t s) {
  quant_rows_kernel<NCH, SUB><<<(rows + 3) / 4, 256, 0, s>>>(a, rows, cols, lda, q, scale);
  return hipGetLastError();
}

// e4m3fn codes of v[0..n) (n even), each clamped to +-448 first, with the
// quantisers' encoder.
__global__ __launch_bounds__(256) void fp8_encode_kernel(const float* __restrict__ v, uint8_t* __restrict__ out,
                                                         int64_t pairs) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i >= pairs) return;
  const uint32_t p = e4m3_pair(clamp448(v[2 * i]), clamp448(v[2 * i + 1]));
  out[2 * i] = static_cast<uint8_t>(p & 0xFFu);
  out[2 * i + 1] = static_cast<uint8_t>(p >> 8);
}

}  // namespace

int quant_max_cols() { return QMAX; }

hipError_t launch_fp8_encode(const float* v, uint8_t* out, int n, hipStream_t s) {
  if (n < 0 || n % 2) return hipErrorInvalidValue;
  const int64_t pairs = n / 2;
  if (pairs == 0) return hipSuccess;
  fp8_encode_kernel<<<static_cast<unsigned>((pairs + 255) / 256), 256, 0, s>>>(v, out, pairs);
  return hipGetLastError();
}

hipError_t launch_quant_rows(const uint16_t* a, int rows, int cols, int64_t lda, uint8_t* q,
                             float* scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (rows < 0 || cols <= 0 || cols % 8 || cols > QMAX || lda < cols || lda % 8) return hipErrorInvalidValue;
  if (reinterpret_cast<uintptr_t>(a) % 16 || reinterpret_cast<uintptr_t>(q) % 8) return hipErrorInvalidValue;
  const int nch = (cols / 8 + 63) / 64;   // chunks per lane
  if (nch <= 1) return go<1>(a, rows, cols, lda, q, scale, s);
  if (nch <= 2) return go<2>(a, rows, cols, lda, q, scale, s);
  if (nch <= 4) return go<4>(a, rows, cols, lda, q, scale, s);
  if (nch <= 8) return go<8>(a, rows, cols, lda, q, scale, s);
  if (nch <= 16) return go<16>(a, rows, cols, lda, q, scale, s);
  return go<32>(a, rows, cols, lda, q, scale, s);
}

hipError_t launch_quant_rows_sub(const uint16_t* a, int rows, int cols, int64_t lda, uint8_t* q,
                                 float* scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (rows < 0 || cols <= 0 || cols % kSubChannel || cols > QMAX || lda < cols || lda % 8)
    return hipErrorInvalidValue;
  if (reinterpret_cast<uintptr_t>(a) % 16 || reinterpret_cast<uintptr_t>(q) % 8) return hipErrorInvalidValue;
  const int nch = cols / kSubChannel;     // chunks per lane = slices
  if (nch <= 1) return go<1, true>(a, rows, cols, lda, q, scale, s);
  if (nch <= 2) return go<2, true>(a, rows, cols, lda, q, scale, s);
  if (nch <= 4) return go<4, true>(a, rows, cols, lda, q, scale, s);
  if (nch <= 8) return go<8, true>(a, rows, cols, lda, q, scale, s);
  if (nch <= 16) return go<16, true>(a, rows, cols, lda, q, scale, s);
  return go<32, true>(a, rows, cols, lda, q, scale, s);
}

hipError_t launch_quant_rows_mx(const uint16_t* a, int rows, int cols, int64_t lda, uint8_t* q,
                                uint8_t* scale, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (rows < 0 || cols <= 0 || cols % 128 || cols > QMAX || lda < cols || lda % 8) return hipErrorInvalidValue;
  if (reinterpret_cast<uintptr_t>(a) % 16 || reinterpret_cast<uintptr_t>(q) % 8) return hipErrorInvalidValue;
  const int nch = (cols / 8 + 63) / 64;
  if (nch <= 1) return go_mx<1>(a, rows, cols, lda, q, scale, s);
  if (nch <= 2) return go_mx<2>(a, rows, cols, lda, q, scale, s);
  if (nch <= 4) return go_mx<4>(a, rows, cols, lda, q, scale, s);
  if (nch <= 8) return go_mx<8>(a, rows, cols, lda, q, scale, s);
  if (nch <= 16) return go_mx<16>(a, rows, cols, lda, q, scale, s);
  return go_mx<32>(a, rows, cols, lda, q, scale, s);
}

}  // namespace moe
