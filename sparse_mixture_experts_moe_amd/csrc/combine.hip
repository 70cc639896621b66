// Unpermute and routing-weighted combine plus the shared branch:
//   y[t] = sum_{j<k} w[t,j] * o_perm[row_of_slot[t*k+j]] + shared[t]
// ("finalize routing" on the "CANN Qwen3-MoE" page; the unpermute and local
// reduce of the "Qwen 3.5 MoE on Ironwood" page's MoE track, which reads each
// expert output row once and writes each token row once).  One block per (token
// row, 1024-column chunk), so a small batch still spreads over the whole GPU;
// every thread owns 8 consecutive hidden elements (16-byte accesses in bf16),
// accumulates in fp32 in slot order (a fused multiply-add per slot, the
// shared row added last) and rounds once.  A token's column chunks
// are consecutive blocks, so the blocks in flight read whole expert rows.
#include <algorithm>

#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int THREADS = 128;
constexpr int CHUNK = THREADS * 8;   // hidden elements per block
constexpr int MAXK = 32;

// 8 elements as stored (bf16: 16 bytes; fp32: 32 bytes), loaded without use
// so that several rows' loads can be in flight together.  bf16 rows are read
// with the non-temporal hint: every expert row is read exactly once (Ling
// prefill combine 0.519 -> 0.462 ms; the next layer's router, reading x right
// after, 107 -> 122 us; layer 14.33 -> 14.25 ms).
typedef unsigned u32x4v __attribute__((ext_vector_type(4)));
template <int DT> struct Raw8;
template <> struct Raw8<DT_BF16> { uint4 q; };
template <> struct Raw8<DT_F32> { float4 a, b; };

template <int DT>
__device__ __forceinline__ Raw8<DT> load_raw(const void* base, int64_t off) {
  Raw8<DT> r;
  if constexpr (DT == DT_BF16) {
    const u32x4v v =
        __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(static_cast<const uint16_t*>(base) + off));
    r.q = uint4{v[0], v[1], v[2], v[3]};
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    r.a = p[0];
    r.b = p[1];
  }
  return r;
}

template <int DT>
__device__ __forceinline__ void widen(const Raw8<DT>& r, float (&v)[8]) {
  if constexpr (DT == DT_BF16) {
    const uint32_t w[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
    v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
  }
}

template <int DT>
__device__ __forceinline__ void store8(void* base, int64_t off, const float (&v)[8]) {
  if constexpr (DT == DT_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = static_cast<uint32_t>(f32_to_bf16(v[2 * i])) |
             (static_cast<uint32_t>(f32_to_bf16(v[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = uint4{w[0], w[1], w[2], w[3]};
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
    p[0] = float4{v[0], v[1], v[2], v[3]};
    p[1] = float4{v[4], v[5], v[6], v[7]};
  }
}

template <int DT>
__global__ __launch_bounds__(THREADS) void combine_kernel(const void* __restrict__ o_perm,
                                                          const int32_t* __restrict__ row_of_slot,
                                                          const float* __restrict__ w,
                                                          const void* __restrict__ shared, int T,
                                                          int D, int k, void* __restrict__ y) {
  __shared__ int32_t rows[MAXK];
  __shared__ float ws[MAXK];
  const int nch = (D + CHUNK - 1) / CHUNK;
  const int t = static_cast<int>(blockIdx.x / nch);
  const int chunk = static_cast<int>(blockIdx.x - static_cast<unsigned>(t) * nch);
  if (threadIdx.x < k) {
    // rows outside [0, T*k) are dropped assignments
    const int32_t r = row_of_slot[static_cast<int64_t>(t) * k + threadIdx.x];
    rows[threadIdx.x] = (r >= 0 && r < static_cast<int64_t>(T) * k) ? r : -1;
    ws[threadIdx.x] = w[static_cast<int64_t>(t) * k + threadIdx.x];
  }
  __syncthreads();
  {
    const int d = chunk * CHUNK + threadIdx.x * 8;
    if (d >= D) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    Raw8<DT> sraw;
    if (shared) sraw = load_raw<DT>(shared, static_cast<int64_t>(t) * D + d);
    // slots in groups of 8: all of a group's loads are issued before the
    // first is used (a slot past k or without a row reads row 0 and is
    // skipped), then the rows are added in slot order
    for (int j0 = 0; j0 < k; j0 += 8) {
      Raw8<DT> raw[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        const int r = j < k ? rows[j] : -1;
        raw[u] = load_raw<DT>(o_perm, static_cast<int64_t>(r < 0 ? 0 : r) * D + d);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        if (j < k && rows[j] >= 0) {
          float v[8];
          widen<DT>(raw[u], v);
          const float wj = ws[j];
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wj, v[i], acc[i]);
        }
      }
    }
    if (shared) {
      float sv[8];
      widen<DT>(sraw, sv);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += sv[i];
    }
    store8<DT>(y, static_cast<int64_t>(t) * D + d, acc);
  }
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t v) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) p[i] = v;
}

}  // namespace

hipError_t launch_fill_i32(int32_t* p, int64_t n, int32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  fill_i32_kernel<<<static_cast<unsigned>(blocks), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

hipError_t launch_combine(const void* o_perm, const int32_t* row_of_slot, const float* w,
                          const void* shared, int T, int D, int k, int dtype, void* y,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int nch = (D + CHUNK - 1) / CHUNK;
  const dim3 grid(static_cast<unsigned>(static_cast<int64_t>(T) * nch));   // T * D < 2^31
  if (dtype == DT_BF16)
    combine_kernel<DT_BF16><<<grid, THREADS, 0, s>>>(o_perm, row_of_slot, w, shared, T, D, k, y);
  else
    combine_kernel<DT_F32><<<grid, THREADS, 0, s>>>(o_perm, row_of_slot, w, shared, T, D, k, y);
  return hipGetLastError();
}

}  // namespace moe
