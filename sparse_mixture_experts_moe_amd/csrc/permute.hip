// Deterministic expert-major permutation of the (token, slot) assignments and
// the per-expert M-tile table of the grouped GEMM.
//
// Counts, their prefix sum and the stable order ("init routing" and "compute
// expert tokens" on the "CANN Qwen3-MoE" page; the contiguous permuted buffer
// that the SparseCore gather of the "Qwen 3.5 MoE on Ironwood" page writes) are
// built without order-dependent atomics:
//   1. each block of PB tokens sets, in LDS, one bit per (expert, token) pair;
//      a token's rank inside its expert is the popcount of the bits of lower
//      tokens, and the block's count is the popcount of the whole mask;
//   2. one block scans the per-block counts down each expert column (each
//      block's first row within the expert) and across experts (exclusive:
//      the expert's first row, its offset);
//   3. every assignment writes row = offset + the block's first row + rank.
// Rows of one expert are therefore in ascending token order.
#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int PB = 256;                 // tokens per permutation block
constexpr int WORDS = PB / 64;          // 64-bit mask words per expert
constexpr int SCAN_THREADS = 1024;      // E <= 1024

__global__ __launch_bounds__(PB) void perm_mask_kernel(const int32_t* __restrict__ idx, int T,
                                                       int k, int E, int32_t* __restrict__ blk,
                                                       int32_t* __restrict__ local_rank) {
  extern __shared__ unsigned long long mask[];  // [E][WORDS]
  for (int i = threadIdx.x; i < E * WORDS; i += PB) mask[i] = 0ull;
  __syncthreads();
  const int tl = threadIdx.x;
  const int t = blockIdx.x * PB + tl;
  const int w = tl >> 6;
  const unsigned long long bit = 1ull << (tl & 63);
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[static_cast<int64_t>(t) * k + j];
      if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) atomicOr(&mask[e * WORDS + w], bit);
    }
  }
  __syncthreads();
  if (t < T) {
    for (int j = 0; j < k; ++j) {
      const int e = idx[static_cast<int64_t>(t) * k + j];
      int r = 0;
      if (static_cast<unsigned>(e) < static_cast<unsigned>(E)) {
        for (int ww = 0; ww < w; ++ww) r += __popcll(mask[e * WORDS + ww]);
        r += __popcll(mask[e * WORDS + w] & (bit - 1ull));
      }
      local_rank[static_cast<int64_t>(t) * k + j] = r;
    }
  }
  for (int e = threadIdx.x; e < E; e += PB) {
    int c = 0;
#pragma unroll
    for (int ww = 0; ww < WORDS; ++ww) c += __popcll(mask[e * WORDS + ww]);
    blk[static_cast<int64_t>(blockIdx.x) * E + e] = c;
  }
}

// Single block: column scans of the per-block counts (turned in place into
// each block's first row within the expert), counts, and the exclusive scan
// over experts (the scatter adds offsets[e]).
__global__ __launch_bounds__(SCAN_THREADS) void perm_scan_kernel(int32_t* __restrict__ blk, int nb,
                                                                 int E, int32_t* __restrict__ counts,
                                                                 int32_t* __restrict__ offsets) {
  __shared__ int32_t sc[SCAN_THREADS];
  const int e = threadIdx.x;
  int run = 0;
  if (e < E) {
    constexpr int NB = 16;   // counts loaded before any is replaced
    for (int b0 = 0; b0 < nb; b0 += NB) {
      int c[NB];
#pragma unroll
      for (int u = 0; u < NB; ++u)
        c[u] = b0 + u < nb ? blk[static_cast<int64_t>(b0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < NB; ++u)
        if (b0 + u < nb) {
          blk[static_cast<int64_t>(b0 + u) * E + e] = run;
          run += c[u];
        }
    }
    counts[e] = run;
  }
  sc[e] = e < E ? run : 0;
  __syncthreads();
  // Hillis-Steele inclusive scan over the expert totals
  for (int off = 1; off < SCAN_THREADS; off <<= 1) {
    const int add = e >= off ? sc[e - off] : 0;
    __syncthreads();
    sc[e] += add;
    __syncthreads();
  }
  const int excl = sc[e] - (e < E ? run : 0);
  if (e < E) {
    offsets[e] = excl;
    if (e == E - 1) offsets[E] = sc[e];
  }
}

__global__ __launch_bounds__(256) void perm_scatter_kernel(const int32_t* __restrict__ idx,
                                                           const int32_t* __restrict__ local_rank,
                                                           const int32_t* __restrict__ blk,
                                                           const int32_t* __restrict__ offsets, int T,
                                                           int k, int E,
                                                           int32_t* __restrict__ row_token,
                                                           int32_t* __restrict__ row_of_slot) {
  const int64_t a = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (a >= static_cast<int64_t>(T) * k) return;
  const int t = static_cast<int>(a / k);
  const int e = idx[a];
  if (static_cast<unsigned>(e) >= static_cast<unsigned>(E)) {
    row_of_slot[a] = -1;
    return;
  }
  const int r = offsets[e] + blk[static_cast<int64_t>(t / PB) * E + e] + local_rank[a];
  row_token[r] = t;
  row_of_slot[a] = r;
}

// Position of group g (< G) in a fixed stride permutation of the groups: a
// stride of about G / 2, made coprime to G, so neighbouring groups land far
// apart in the order.  (Odd start, steps of 2: the search reaches a unit mod
// G, so it ends.)
__device__ __forceinline__ int spread_rank(int g, int G) {
  int a = (G / 2 + 1) | 1;
  for (;;) {
    int x = a, y = G;
    while (y) {
      const int t = x % y;
      x = y;
      y = t;
    }
    if (x == 1) break;
    a += 2;
  }
  return static_cast<int>((static_cast<int64_t>(g) * a) % G);
}

// Single block: each group's M-tiles.  With largest_first the groups are
// ordered by descending row count (ties by group id) so the heaviest experts
// start first; otherwise in group order.  With tiles2, a second table of
// bm2-row tiles in the same group order (one ranking, one scan for both).
constexpr int TILE_THREADS = 1024;

__device__ __forceinline__ int clamp_row(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

__global__ __launch_bounds__(TILE_THREADS) void build_tiles_kernel(const int32_t* __restrict__ offsets,
                                                                   int G, int bm, int max_rows,
                                                                   int max_tiles, int largest_first,
                                                                   GTile* __restrict__ tiles,
                                                                   int32_t* __restrict__ n_tiles, int bm2,
                                                                   int max_tiles2,
                                                                   GTile* __restrict__ tiles2,
                                                                   int32_t* __restrict__ n_tiles2) {
  __shared__ int32_t sz[TILE_THREADS];    // group sizes (offsets clamped to [0, max_rows])
  __shared__ int32_t ntl[TILE_THREADS];   // tiles of the group at each rank position
  __shared__ int32_t ntl2[TILE_THREADS];  // the same for the second table
  __shared__ int32_t grp[TILE_THREADS];   // group at each rank position
  const int g = threadIdx.x;
  int r0 = 0, n = 0;
  if (g < G) {
    r0 = clamp_row(offsets[g], 0, max_rows);
    n = clamp_row(offsets[g + 1], r0, max_rows) - r0;
  }
  sz[g] = n;
  __syncthreads();
  int rank = g;
  if (largest_first && g < G) {
    rank = 0;
    for (int o = 0; o < G; ++o) {
      const int no = sz[o];
      rank += (no > n) || (no == n && o < g);
    }
  }
  const bool two = tiles2 != nullptr;
  ntl[g] = 0;
  ntl2[g] = 0;
  __syncthreads();
  if (g < G) {
    ntl[rank] = (n + bm - 1) / bm;
    if (two) ntl2[rank] = (n + bm2 - 1) / bm2;
    grp[rank] = g;
  }
  __syncthreads();
  // inclusive scans of tile counts in rank order
  for (int off = 1; off < TILE_THREADS; off <<= 1) {
    const int add = g >= off ? ntl[g - off] : 0;
    const int add2 = g >= off ? ntl2[g - off] : 0;
    __syncthreads();
    ntl[g] += add;
    ntl2[g] += add2;
    __syncthreads();
  }
  auto write = [&](GTile* tl_out, const int32_t* sc, int tb, int cap) {
    const int gg = grp[g];
    const int a = clamp_row(offsets[gg], 0, max_rows);
    const int b = a + sz[gg];
    const int base = g > 0 ? sc[g - 1] : 0;
    for (int i = 0, r = a; r < b && base + i < cap; ++i, r += tb) {
      GTile tl;
      tl.group = gg;
      tl.row0 = r;
      tl.row1 = r + tb < b ? r + tb : b;
      tl.pad = 0;
      tl_out[base + i] = tl;
    }
  };
  if (g < G) {
    write(tiles, ntl, bm, max_tiles);
    if (two) write(tiles2, ntl2, bm2, max_tiles2);
  }
  if (g == 0) {
    const int total = G > 0 ? ntl[G - 1] : 0;
    n_tiles[0] = total < max_tiles ? total : max_tiles;
    if (two) {
      const int total2 = G > 0 ? ntl2[G - 1] : 0;
      n_tiles2[0] = total2 < max_tiles2 ? total2 : max_tiles2;
    }
  }
}

// Batches of at most 1024 tokens (decode): the whole permutation and the
// M-tile table (in group order) in one block, with the same bit-mask ranking.
__device__ __forceinline__ int block_inclusive_scan(int32_t* sc, int v) {
  const int i = threadIdx.x;
  sc[i] = v;
  __syncthreads();
  for (int off = 1; off < SCAN_THREADS; off <<= 1) {
    const int add = i >= off ? sc[i - off] : 0;
    __syncthreads();
    sc[i] += add;
    __syncthreads();
  }
  return sc[i];
}

// MW 64-bit mask words per expert: batches of at most 64 * MW tokens.
template <int MW>
__global__ __launch_bounds__(SCAN_THREADS) void perm_small_kernel(
    const int32_t* __restrict__ idx, int T, int k, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ row_token, int32_t* __restrict__ row_of_slot,
    int bm, int max_tiles, int spread, GTile* __restrict__ tiles, int32_t* __restrict__ n_tiles) {
  constexpr int WORDS = MW;
  __shared__ unsigned long long mask[SCAN_THREADS * WORDS];   // [E][WORDS]
  __shared__ int32_t sc[SCAN_THREADS];
  __shared__ int32_t off_s[SCAN_THREADS + 1];
  const int tid = threadIdx.x;
  for (int i = tid; i < E * WORDS; i += SCAN_THREADS) mask[i] = 0ull;
  __syncthreads();
  const int n = T * k;
  for (int a = tid; a < n; a += SCAN_THREADS) {
    const int t = a / k, e = idx[a];
    if (static_cast<unsigned>(e) < static_cast<unsigned>(E))
      atomicOr(&mask[e * WORDS + (t >> 6)], 1ull << (t & 63));
  }
  __syncthreads();
  int c = 0;
  if (tid < E) {
#pragma unroll
    for (int w = 0; w < WORDS; ++w) c += __popcll(mask[tid * WORDS + w]);
    counts[tid] = c;
  }
  const int incl = block_inclusive_scan(sc, tid < E ? c : 0);
  if (tid < E) {
    off_s[tid] = incl - c;
    offsets[tid] = incl - c;
    if (tid == E - 1) {
      off_s[E] = incl;
      offsets[E] = incl;
    }
  }
  __syncthreads();
  for (int a = tid; a < n; a += SCAN_THREADS) {
    const int t = a / k, e = idx[a];
    if (static_cast<unsigned>(e) >= static_cast<unsigned>(E)) {
      row_of_slot[a] = -1;
      continue;
    }
    int r = off_s[e];
    const int w = t >> 6;
    for (int ww = 0; ww < w; ++ww) r += __popcll(mask[e * WORDS + ww]);
    r += __popcll(mask[e * WORDS + w] & ((1ull << (t & 63)) - 1ull));
    row_token[r] = t;
    row_of_slot[a] = r;
  }
  if (!tiles) return;
  // M-tiles of each group: groups in id order or, spread, in a fixed stride
  // order that puts neighbouring groups far apart (measured faster than
  // largest-first here: blocks that run together then stream weights from
  // experts far apart)
  __shared__ int32_t sz[SCAN_THREADS];
  __shared__ int32_t grp[SCAN_THREADS];
  sz[tid] = tid < E ? c : 0;
  __syncthreads();
  int rank = tid;
  if (spread && tid < E) rank = spread_rank(tid, E);
  if (tid < E) grp[rank] = tid;
  __syncthreads();
  const int gg = tid < E ? grp[tid] : 0;           // group at rank position tid
  const int nt = tid < E ? (sz[gg] + bm - 1) / bm : 0;
  const int tincl = block_inclusive_scan(sc, nt);
  if (tid < E) {
    const int base = tincl - nt;
    for (int i = 0; i < nt && base + i < max_tiles; ++i) {
      GTile tl;
      tl.group = gg;
      tl.row0 = off_s[gg] + i * bm;
      tl.row1 = min(off_s[gg] + (i + 1) * bm, off_s[gg + 1]);
      tl.pad = 0;
      tiles[base + i] = tl;
    }
  }
  if (tid == SCAN_THREADS - 1) n_tiles[0] = min(tincl, max_tiles);
}

// The materialised permuted copy ("Qwen 3.5 MoE on Ironwood", MoE track: the
// gather of the routed tokens into one contiguous buffer): row r of x_perm is
// x[row_token[r]], for the rows the permutation filled (r < offsets[E]).  One
// block per sorted row, 16-byte copies.
__global__ __launch_bounds__(256) void gather_rows_kernel(const char* __restrict__ x,
                                                          const int32_t* __restrict__ row_token,
                                                          const int32_t* __restrict__ n_rows, int T,
                                                          int64_t row_bytes, char* __restrict__ x_perm) {
  const int r = blockIdx.x;
  if (r >= n_rows[0]) return;
  const int t = row_token[r];
  if (static_cast<unsigned>(t) >= static_cast<unsigned>(T)) return;   // not filled by the permutation
  const uint4* src = reinterpret_cast<const uint4*>(x + static_cast<int64_t>(t) * row_bytes);
  uint4* dst = reinterpret_cast<uint4*>(x_perm + static_cast<int64_t>(r) * row_bytes);
  for (int64_t i = threadIdx.x; i < row_bytes / 16; i += blockDim.x) dst[i] = src[i];
}

}  // namespace

int perm_blocks(int T) { return static_cast<int>((static_cast<int64_t>(T) + PB - 1) / PB); }

int perm_small_max_tokens() { return 16 * 64; }

hipError_t launch_permute_small(const int32_t* idx, int T, int k, int E, int32_t* counts,
                                int32_t* offsets, int32_t* row_token, int32_t* row_of_slot, int bm,
                                int max_tiles, bool spread, GTile* tiles, int32_t* n_tiles,
                                hipStream_t s) {
  if (T > perm_small_max_tokens()) return hipErrorInvalidValue;
  const int lf = spread ? 1 : 0;
  if (T <= 4 * 64)
    perm_small_kernel<4><<<1, SCAN_THREADS, 0, s>>>(idx, T, k, E, counts, offsets, row_token,
                                                    row_of_slot, bm, max_tiles, lf, tiles, n_tiles);
  else if (T <= 8 * 64)
    perm_small_kernel<8><<<1, SCAN_THREADS, 0, s>>>(idx, T, k, E, counts, offsets, row_token,
                                                    row_of_slot, bm, max_tiles, lf, tiles, n_tiles);
  else
    perm_small_kernel<16><<<1, SCAN_THREADS, 0, s>>>(idx, T, k, E, counts, offsets, row_token,
                                                     row_of_slot, bm, max_tiles, lf, tiles, n_tiles);
  return hipGetLastError();
}

hipError_t launch_permute(const int32_t* idx, int T, int k, int E, int32_t* blk, int32_t* local_rank,
                          int32_t* counts, int32_t* offsets, int32_t* row_token,
                          int32_t* row_of_slot, hipStream_t s) {
  const int nb = perm_blocks(T);
  if (nb > 0) {
    perm_mask_kernel<<<nb, PB, sizeof(unsigned long long) * WORDS * E, s>>>(idx, T, k, E, blk,
                                                                           local_rank);
  }
  perm_scan_kernel<<<1, SCAN_THREADS, 0, s>>>(blk, nb, E, counts, offsets);
  const int64_t n = static_cast<int64_t>(T) * k;
  if (n > 0) {
    perm_scatter_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, s>>>(
        idx, local_rank, blk, offsets, T, k, E, row_token, row_of_slot);
  }
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* x, const int32_t* row_token, const int32_t* n_rows, int T,
                              int rows, int64_t row_bytes, void* x_perm, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int threads = row_bytes / 16 >= 256 ? 256 : 64;
  gather_rows_kernel<<<rows, threads, 0, s>>>(static_cast<const char*>(x), row_token, n_rows, T, row_bytes,
                                              static_cast<char*>(x_perm));
  return hipGetLastError();
}

hipError_t launch_build_tiles(const int32_t* offsets, int n_groups, int bm, int max_rows,
                              int max_tiles, bool largest_first, GTile* tiles, int32_t* n_tiles,
                              hipStream_t s) {
  build_tiles_kernel<<<1, TILE_THREADS, 0, s>>>(offsets, n_groups, bm, max_rows, max_tiles,
                                                largest_first ? 1 : 0, tiles, n_tiles, 0, 0, nullptr,
                                                nullptr);
  return hipGetLastError();
}

hipError_t launch_build_tiles_pair(const int32_t* offsets, int n_groups, int max_rows,
                                   bool largest_first, int bm, int max_tiles, GTile* tiles,
                                   int32_t* n_tiles, int bm2, int max_tiles2, GTile* tiles2,
                                   int32_t* n_tiles2, hipStream_t s) {
  if (!tiles2 || bm2 <= 0) return hipErrorInvalidValue;
  build_tiles_kernel<<<1, TILE_THREADS, 0, s>>>(offsets, n_groups, bm, max_rows, max_tiles,
                                                largest_first ? 1 : 0, tiles, n_tiles, bm2,
                                                max_tiles2, tiles2, n_tiles2);
  return hipGetLastError();
}

}  // namespace moe
