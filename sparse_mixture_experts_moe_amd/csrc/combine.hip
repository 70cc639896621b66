// Unpermute and routing-weighted combine plus the shared branch:
//   y[t] = sum_{j<k} w[t,j] * o_perm[row_of_slot[t*k+j]] + shared[t]
// ("finalize routing" on the "CANN Qwen3-MoE" page; the unpermute and local
// reduce of the "Qwen 3.5 MoE on Ironwood" page's MoE track, which reads each
// expert output row once and writes each token row once).  One block per (token
// row, 1024-column chunk), so a small batch still spreads over the whole GPU;
// every thread owns 8 consecutive hidden elements (16-byte accesses in bf16),
// accumulates in fp32 in slot order and rounds once.
#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int THREADS = 128;
constexpr int CHUNK = THREADS * 8;   // hidden elements per block
constexpr int MAXK = 32;

template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t off, float (&v)[8]) {
  if constexpr (DT == DT_BF16) {
    const uint4 q = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    const float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
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
                                                          const void* __restrict__ shared, int D,
                                                          int k, void* __restrict__ y) {
  __shared__ int32_t rows[MAXK];
  __shared__ float ws[MAXK];
  const int t = blockIdx.x;
  if (threadIdx.x < k) {
    rows[threadIdx.x] = row_of_slot[static_cast<int64_t>(t) * k + threadIdx.x];
    ws[threadIdx.x] = w[static_cast<int64_t>(t) * k + threadIdx.x];
  }
  __syncthreads();
  {
    const int d = blockIdx.y * CHUNK + threadIdx.x * 8;
    if (d >= D) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int r = rows[j];
      if (r < 0) continue;
      float v[8];
      load8<DT>(o_perm, static_cast<int64_t>(r) * D + d, v);
      const float wj = ws[j];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += wj * v[i];
    }
    if (shared) {
      float v[8];
      load8<DT>(shared, static_cast<int64_t>(t) * D + d, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    store8<DT>(y, static_cast<int64_t>(t) * D + d, acc);
  }
}

}  // namespace

hipError_t launch_combine(const void* o_perm, const int32_t* row_of_slot, const float* w,
                          const void* shared, int T, int D, int k, int dtype, void* y,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  const dim3 grid(T, (D + CHUNK - 1) / CHUNK);
  if (dtype == DT_BF16)
    combine_kernel<DT_BF16><<<grid, THREADS, 0, s>>>(o_perm, row_of_slot, w, shared, D, k, y);
  else
    combine_kernel<DT_F32><<<grid, THREADS, 0, s>>>(o_perm, row_of_slot, w, shared, D, k, y);
  return hipGetLastError();
}

}  // namespace moe
