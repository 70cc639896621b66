// Top-k softmax gating, one 64-wide wavefront per token.
//
// Selection is an exact comparison of fp32 logits: k rounds of a wavefront
// arg-max over (value, -expert) keys, so equal values go to the lower expert
// index (+0 and -0 compare equal).  The weights are the renormalised top-k of
// the softmax, w_j = exp(l_j - l_0) / sum_m exp(l_m - l_0), which is the fused
// top-k softmax of the "CANN Qwen3-MoE" page (GMM enablement and routing
// optimisation) and the softmax-then-top-10 router of the "Qwen 3.5 MoE on
// Ironwood" page (model architecture) after renormalisation; or, without
// renormalisation, the selected experts' softmax probabilities over all
// experts (the router as a linear layer plus softmax, "TP MoE" page, 3.3).
#include "moe_kernels.h"

namespace moe {
namespace {

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// k rounds of a wavefront arg-max over the lane's EPL logits v (expert
// lane + 64 j), then the weights; lane r < k stores slot r of token t.
template <int EPL>
__device__ __forceinline__ void select_topk(const float (&v)[EPL], int lane, int t, int E, int k,
                                            int renorm, int32_t* __restrict__ idx,
                                            float* __restrict__ wout) {
  uint32_t taken = 0;
  float my_v = 0.f, top_v = 0.f;
  int my_i = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -__builtin_inff();
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      if (e < E && !(taken >> j & 1u) && better(v[j], e, bv, bi)) {
        bv = v[j];
        bi = e;
      }
    }
    // butterfly arg-max: every lane ends with the wavefront's best key
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 64);
      const int oi = __shfl_xor(bi, off, 64);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (r == 0) top_v = bv;
    if (lane == r) {
      my_v = bv;
      my_i = bi;
    }
  }
  float ex = lane < k ? expf(my_v - top_v) : 0.f;
  // denominator: the k selected terms (renormalised), or every expert's term
  // (plain softmax probabilities); lane partial sums in a fixed order, then a
  // butterfly, so the result does not depend on scheduling
  float sum = ex;
  if (!renorm) {
    sum = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (lane + 64 * j < E) sum += expf(v[j] - top_v);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  if (lane < k) {
    idx[static_cast<int64_t>(t) * k + lane] = my_i;
    wout[static_cast<int64_t>(t) * k + lane] = ex / sum;
  }
}


// One block per token.  The router product may arrive as `splits` partial sums
// (a K-split GEMM): all threads of the block add them in slice order into LDS
// (so the logits are deterministic), then wavefront 0 selects the top k.
// Used for many partial sums (a decode batch's router).
template <int EPL, int TOPK_THREADS>
__global__ __launch_bounds__(TOPK_THREADS) void topk_softmax_kernel(
    const float* __restrict__ part, int splits, float* __restrict__ logits_out, int T, int E,
    int k, int renorm, int32_t* __restrict__ idx, float* __restrict__ wout) {
  __shared__ float lg[64 * EPL];
  const int t = blockIdx.x;
  const int64_t slice = static_cast<int64_t>(T) * E;
  const float* row = part + static_cast<int64_t>(t) * E;
  for (int e = threadIdx.x; e < E; e += TOPK_THREADS) {
    float l = row[e];
    for (int s0 = 1; s0 < splits; s0 += 8) {
      float pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) pv[u] = s0 + u < splits ? row[(s0 + u) * slice + e] : 0.f;
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u < splits) l += pv[u];
    }
    lg[e] = l;
    if (logits_out) logits_out[static_cast<int64_t>(t) * E + e] = l;
  }
  __syncthreads();
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  float v[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? lg[e] : -__builtin_inff();
  }
  select_topk<EPL>(v, lane, t, E, k, renorm, idx, wout);
}

// Few partial sums (at most kWaveSplits): one wavefront per token, four tokens
// per block, each lane adding its experts' partial sums in slice order (the
// same additions as above), so every wavefront selects at once.
constexpr int kWaveSplits = 4;
template <int EPL>
__global__ __launch_bounds__(256) void topk_softmax_wave_kernel(
    const float* __restrict__ part, int splits, float* __restrict__ logits_out, int T, int E,
    int k, int renorm, int32_t* __restrict__ idx, float* __restrict__ wout) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const int64_t slice = static_cast<int64_t>(T) * E;
  const float* row = part + static_cast<int64_t>(t) * E;
  float v[EPL];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? row[e] : -__builtin_inff();
  }
  // every slice's loads first, then the additions in slice order
  float pv[kWaveSplits - 1][EPL];
#pragma unroll
  for (int s0 = 1; s0 < kWaveSplits; ++s0)
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      pv[s0 - 1][j] = (s0 < splits && e < E) ? row[s0 * slice + e] : 0.f;
    }
#pragma unroll
  for (int s0 = 1; s0 < kWaveSplits; ++s0)
    if (s0 < splits) {
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if (lane + 64 * j < E) v[j] += pv[s0 - 1][j];
    }
  if (logits_out) {
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const int e = lane + 64 * j;
      if (e < E) logits_out[static_cast<int64_t>(t) * E + e] = v[j];
    }
  }
  select_topk<EPL>(v, lane, t, E, k, renorm, idx, wout);
}

template <int EPL>
void go(const float* part, int splits, float* logits_out, int T, int E, int k, int renorm,
        int32_t* idx, float* w, hipStream_t s) {
  if (splits <= kWaveSplits)
    topk_softmax_wave_kernel<EPL><<<(T + 3) / 4, 256, 0, s>>>(part, splits, logits_out, T, E, k,
                                                              renorm, idx, w);
  else
    topk_softmax_kernel<EPL, 256><<<T, 256, 0, s>>>(part, splits, logits_out, T, E, k, renorm,
                                                    idx, w);
}

}  // namespace

hipError_t launch_topk_softmax(const float* part, int splits, float* logits_out, int T, int E,
                               int k, int renorm, int32_t* idx, float* w, hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int epl = (E + 63) / 64;
  if (epl <= 1) go<1>(part, splits, logits_out, T, E, k, renorm, idx, w, s);
  else if (epl <= 2) go<2>(part, splits, logits_out, T, E, k, renorm, idx, w, s);
  else if (epl <= 4) go<4>(part, splits, logits_out, T, E, k, renorm, idx, w, s);
  else if (epl <= 8) go<8>(part, splits, logits_out, T, E, k, renorm, idx, w, s);
  else go<16>(part, splits, logits_out, T, E, k, renorm, idx, w, s);
  return hipGetLastError();
}

}  // namespace moe
