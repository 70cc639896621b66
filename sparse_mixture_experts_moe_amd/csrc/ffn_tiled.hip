// LDS-tiled grouped GEMM: prefill-sized groups, and decode batches in a
// 32-row shape.
//
// Prefill is bound by the MFMA units once every expert has hundreds of rows
// ("Qwen 3.5 MoE on Ironwood", roofline section: prefill is compute-bound and
// uneven expert loads make padding in the grouped GEMM the thing to minimise;
// "Ling-2.6-1T with SGLang-JAX", section 4: keep tokens and accumulators
// resident and stream the expert weights with the next tile's fetch in flight).
//
// Block tile: BM sorted rows of one group x BNW weight rows, in four shapes:
// "tall" (256 x 256, 8 wavefronts, one block per CU) for the expert FFNs -- an
// expert's weights are read once per 256 rows, and the row fragments a short
// tile does not fill are skipped --, "wide" (128 x 512, 8 wavefronts) and
// "narrow" (128 x 256, 4 wavefronts, two blocks per CU) for larger groups and
// dense products such as the router, and "small" (32 x 128, 4 wavefronts of
// 32 x 32, two blocks per CU) for decode batches, where the weights only need
// to stream through.  In the first three every SIMD runs two wavefronts of 64
// rows x 128 weight rows (128 accumulators each, in AGPRs), which is what it
// takes to keep the matrix cores busy; 16x16x32 bf16 MFMAs take the weight fragment as the M
// operand, so a lane's accumulator holds 4 consecutive output columns of one
// row.  For the fused gate/up projection the BNW weight rows are BNW/2 gate
// rows and the matching BNW/2 up rows; each wavefront holds the gate and up
// halves of the same 64 h columns and forms act(gate)*up in registers (the
// packed gate/up tile of GMM v2 on the Ironwood page).
//
// K is staged BK elements at a time through a ring of S LDS buffers filled by
// direct HBM -> LDS loads (global_load_lds_dwordx4: a lane's 16 bytes land at
// the instruction's LDS base + 16 x lane).  Stage st+S is fetched while stage
// st is multiplied, and a wavefront's fragments for the next 32-deep sub-step
// are read from LDS while its MFMAs of the current one run, so neither the
// fetch latency nor the LDS latency sits in front of the matrix cores; the
// copies of a stage are spread between the MFMA groups.  One barrier per stage
// publishes a stage's copies and frees the slot that was read before.
//
// Each copy fetches BK contiguous elements of a row, and the L2 serves one
// request per row segment whatever its length, so with fp8 weights (32-byte
// segments at BK = 32) the GEMM is bound by the L2's request rate before the
// matrix cores; fp8 weights are therefore staged 64 deep (64-byte weight and
// 128-byte activation segments, half the requests per FLOP).  bf16 tiles stay
// 32 deep, where a deeper stage would leave fewer than three in the LDS ring.
// The small shape stages 128 deep (256 deep for bf16 weights over a long K),
// so its weight-row requests are 128 to 512 bytes; a stage then spans four or
// eight MFMA sub-steps, its copies spread over them.
//
// Workgroup b runs on XCD b % 8, and each XCD has its own L2: the 256-row
// shape and the bf16-weight 128 x 512 shape map all N blocks of a group of
// consecutive M-tiles to one XCD (groups interleaved across XCDs), so the
// tiles' activation rows are fetched into one L2 and an expert's weight slab
// is shared by its tiles in the group; the other shapes keep N block n of
// every tile on XCD n.
//
// With fp8 activations as well (dynamic per-token quantisation, "Ling-2.6-1T
// with SGLang-JAX" page, section 5: fp8 tokens and fp8 weights straight into
// the matrix unit, per-token and per-channel scales after the reduction) both
// tiles hold e4m3fn bytes, the products are 32x32x64 fp8 MFMAs (twice the
// bf16 rate), stages are 128 deep (128-byte requests for both operands) and
// the epilogue multiplies by the row's activation scale as well.
//
// W4A8 ("CANN Qwen3-MoE" page, high-throughput prefill: MXFP4 weights, MXFP8
// activations): the weight tile holds e2m1 pairs, and each stage also stages
// the E8M0 block scales of its activation rows and weight rows (4 bytes per
// row per 128-deep stage), which the scaled MFMA applies per 32-element block.
// Fragments follow the matrix unit's own K order so that each of its two
// scale blocks per MFMA is exactly one MX block.
//
// A tile row of RB bytes holds RB / 16 chunks of 16 bytes; chunk c of row r
// sits at a position XORed with a few bits of r (upos below), chosen so that
// the rows sharing a 256-byte line of the 64 banks, and the rows one fragment
// read serves per cycle, fall on distinct banks.  Since a copy lane's LDS
// position is fixed by its lane index, the swizzle is applied on the source
// side: the lane that fills a position fetches the chunk that belongs there.
// fp8 e4m3fn weights stay fp8 in LDS and are decoded exactly to bf16 when a
// sub-step's fragments are taken up, which halves the weight tile's LDS
// footprint; per-channel scales are applied after the reduction.
#include <type_traits>

#include "moe_kernels.h"

namespace moe {
namespace {

constexpr int KS = 32;                    // K elements per MFMA sub-step
constexpr int BK8A = 128;                 // stage depth of fp8 x fp8 tiles (64 measured 6 % slower)
constexpr int LDS_CU = 160 * 1024;        // LDS per CU

template <int BM_, int BNW_, int WM_, int WN_, int BPC_, bool FP8, int BK_, int MF_, bool A8_ = false,
          bool W4_ = false, bool SUB_ = false>
struct Cfg {
  static constexpr bool A8 = A8_;                     // fp8 activations (with fp8 weights)
  static constexpr bool W4 = W4_;                     // MXFP4 weights, MXFP8 activations (with A8)
  static constexpr bool SUB = SUB_;                   // fp8 activations with sub-channel scales (with A8)
  static constexpr bool W8 = FP8;                     // one-byte weights (fp8, or e2m1 pairs with W4)
  static constexpr int MF = MF_;                      // MFMA tile: 16 (16x16x32) or 32 (32x32x16 / x64 fp8)
  static constexpr int BK = BK_;                      // K elements per stage
  static constexpr int KSUB = A8 ? 64 : KS;           // K elements per MFMA sub-step
  static constexpr int H = BK / KSUB;                 // sub-steps per stage
  static constexpr int ROWB = BK * 2;                 // LDS bytes per bf16 tile row
  static constexpr int ROWB8 = BK;                    // LDS bytes per fp8 tile row
  static constexpr int ROWA = A8 ? ROWB8 : ROWB;      // LDS bytes per activation tile row
  static constexpr int BM = BM_;                      // rows per M-tile
  static constexpr int BNW = BNW_;                    // weight rows per block
  static constexpr int WM = WM_, WN = WN_;            // wavefront grid (rows x weights)
  static constexpr int NW = WM * WN;
  static constexpr int THREADS = 64 * NW;
  static constexpr int BPC = BPC_;                    // blocks per CU
  static constexpr int TF = BM / WM / MF;             // MF-row fragments per wavefront
  static constexpr int WF = BNW / WN / MF;            // MF-weight-row fragments per wavefront
  static constexpr int WPE = NW * BPC / 4;            // wavefronts per SIMD
  static constexpr int A_BYTES = BM * ROWA;
  static constexpr int ROWBW = W4 ? BK / 2 : FP8 ? ROWB8 : ROWB;   // LDS bytes per weight tile row
  static constexpr int B_BYTES = BNW * ROWBW;
  // MX block scales of a stage, 4 bytes per row ([row][block]): activation
  // rows one 4-byte copy per lane (gathered rows), weight rows 16 bytes (four
  // consecutive rows) per lane.  Sub-channel scales: the fp32 scale of the
  // stage's slice for each activation row, copied the same way.
  static constexpr int ASC_BYTES = (W4 || SUB) ? BM * 4 : 0;
  static constexpr int BSC_BYTES = W4 ? BNW * 4 : 0;
  static constexpr int ASC_I = ASC_BYTES / 256, BSC_I = BSC_BYTES / 1024;
  static constexpr int NSC = ASC_I + BSC_I;           // scale copy instructions (one per wavefront)
  static constexpr int STAGE = A_BYTES + B_BYTES + ASC_BYTES + BSC_BYTES;
  static constexpr int S0 = LDS_CU / BPC / STAGE;
  static constexpr int S = S0 > 6 ? 6 : S0;           // LDS ring depth
  static constexpr int LDS = S * STAGE;
  static constexpr int AL = A_BYTES / 1024 / NW;      // 1 KiB copy instructions per wavefront, A
  static constexpr int BL = B_BYTES / 1024 / NW;      // same, B
  static constexpr int P = AL + BL;
  static constexpr int P1 = (P + H - 1) / H;          // copies issued per sub-step (the last chunk fewer)
  static_assert(AL * NW * 1024 == A_BYTES && BL * NW * 1024 == B_BYTES, "copy split");
  static_assert(H == 1 || H == 2 || H == 4 || H == 8, "stage depth");
  static_assert(S >= 3 || (S == 2 && H >= 2), "ring depth");
  static_assert(TF * WF * MF * MF / 64 * WPE <= 256, "accumulators fit the AGPRs");
  static_assert(WPE == 1 || WPE == 2, "one or two wavefronts per SIMD");
  static_assert(!A8 || (FP8 && MF == 32), "fp8 activations: fp8 weights, 32x32x64 MFMAs");
  static_assert(!W4 || (A8 && BK == 128), "MX weights: fp8 activations, 128-deep stages");
  static_assert(!SUB || (A8 && !W4 && kSubChannel % BK == 0), "sub-channel scales: whole stages per slice");
  static_assert(ASC_I * 256 == ASC_BYTES && BSC_I * 1024 == BSC_BYTES && NSC <= NW, "scale copies");
};

// position of 16-byte chunk c in a tile row of RB bytes (an involution in c):
// 256 / RB rows share a line of the 64 banks, and consecutive groups of them
// XOR the chunk index with consecutive values
template <int RB> __device__ __forceinline__ int upos(int row, int c) {
  constexpr int SH = RB == 32 ? 3 : RB == 64 ? 2 : RB == 128 ? 1 : 0;
  return c ^ ((row >> SH) & (RB / 16 - 1));
}

// HBM -> LDS copy of 16 bytes per lane from sbase + voff to lds + 16 * lane;
// sbase and lds are wave-uniform.  Issued through inline asm so the compiler
// does not conservatively wait for every copy in flight before each LDS read;
// completion is tracked explicitly with wait_vm below.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(uint32_t voff, const void* sbase, const void* lds) {
  const uint32_t l = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds))));
  const uint64_t b = reinterpret_cast<uint64_t>(sbase);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
  const uint64_t bs = static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(bs), "s"(l)
               : "memory", "m0");
}
// Same with 4 bytes per lane (to lds + 4 * lane).
__device__ __forceinline__ void dma4(uint32_t voff, const void* sbase, const void* lds) {
  const uint32_t l = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds))));
  const uint64_t b = reinterpret_cast<uint64_t>(sbase);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
  const uint64_t bs = static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(bs), "s"(l)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// A wave-uniform pointer, held in scalar registers.
template <class T> __device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v)));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32)));
  return reinterpret_cast<T*>(static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
}

// Wait until at most N of this wavefront's vector-memory operations are in
// flight (they complete in order).
// A sub-channel scale s > 0 as m 2^(e - 127): e the E8M0 code of s's power of
// two (floor(log2 s) kept within [-127, 127]) and m = s / 2^(e - 127), in
// [1, 2) for a normal s; both parts exact.
__device__ __forceinline__ float split_scale(float s, int& e) {
  int ex;
  (void)frexpf(s, &ex);            // s = f 2^ex, f in [0.5, 1)
  const int p = min(127, max(-127, ex - 1));
  e = p + 127;
  return ldexpf(s, -p);
}

template <int N> __device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Wait for all but the newest `newer` groups of P copies (newer <= M).
template <int P, int M> __device__ __forceinline__ void wait_newer(int newer) {
  if constexpr (M == 0) {
    wait_vm<0>();
  } else {
    if (newer >= M) wait_vm<M * P>();
    else wait_newer<P, M - 1>(newer);
  }
}

constexpr int NXCD = 8;       // XCDs; workgroup i is dispatched to XCD i % NXCD
constexpr int XCD_CUS = 32;   // compute units per XCD
// XCD-grouped block order: consecutive M-tiles are taken G at a time, and
// all N blocks of such a group run on one XCD (group j on XCD j % NXCD,
// groups interleaved across the XCDs).  A group's tiles' activation rows are
// then fetched into one L2 instead of eight, and the weight slab of an N
// block is shared by the group's tiles of one expert, which run side by side.
// The 256-row shape takes one tile per group (its experts mostly have one
// tile); the 128 x 512 shape with bf16 weights takes as many tiles as make
// one block per CU of the XCD (Qwen-sized prefill 4.58 -> 4.39 ms).  The
// other shapes keep the launch order (N block n of every tile on XCD n): with
// fp8 weights the grouped order measured slower (Ling-sized prefill 14.40 ->
// 15.04 ms) and fetched no fewer bytes, the blocks of a group drifting apart
// within a few stages.
template <class C> constexpr bool xcdtile() { return C::BM == 256 || (C::BM == 128 && C::BNW == 512 && !C::W8); }
template <class C> __host__ __device__ inline int xcd_tiles(int bpm) {
  return C::BM == 256 || bpm >= XCD_CUS ? 1 : XCD_CUS / bpm;
}

// The XCD-grouped order applies to grids without K slices.
__host__ __device__ inline bool xcdtile_ok(const GArgs& g) {
  for (int i = 0; i < g.nsets; ++i)
    if (g.s[i].ksplit > 1) return false;
  return true;
}
// Physical grid of the XCD-grouped order: each set's tiles padded to a
// multiple of NXCD groups, all of a tile's N blocks.
template <class C> __host__ __device__ inline int xcdtile_grid(const GArgs& g) {
  int n = 0;
  for (int i = 0; i < g.nsets; ++i) {
    const int gt = NXCD * xcd_tiles<C>(g.s[i].blocks_per_m);
    n += (g.s[i].m_slots + gt - 1) / gt * gt * g.s[i].blocks_per_m;
  }
  return n;
}
// Logical block (resolve_block's numbering, tile-major) of physical block b
// in the XCD-grouped order; false if b has no tile.  Block b is the
// (b / NXCD)-th of XCD x = b % NXCD: within a set, XCD x runs groups x,
// x + NXCD, ... in turn, each group's tiles with all their N blocks.
template <class C> __device__ __forceinline__ bool xcdtile_block(const GArgs& g, int b, int& logical) {
  for (int i = 0; i < g.nsets; ++i) {
    const GSet& S = g.s[i];
    const int bpm = S.blocks_per_m;
    const int G = xcd_tiles<C>(bpm);
    const int seg = (S.m_slots + NXCD * G - 1) / (NXCD * G) * (NXCD * G) * bpm;   // a multiple of NXCD
    if (b < seg) {
      const int x = b % NXCD, q = b / NXCD;
      const int grp = x + NXCD * (q / (G * bpm)), e = q % (G * bpm);
      const int tile = grp * G + e / bpm, n = e % bpm;
      if (tile >= S.m_slots) return false;
      logical = S.block0 + tile * bpm + n;
      return true;
    }
    b -= seg;
  }
  return false;
}

// 16 bytes read at device scope (four 4-byte loads that bypass this XCD's
// non-coherent cache lines): rows another XCD's block wrote in this launch.
__device__ __forceinline__ uint4 load16_device(const uint16_t* p) {
  uint32_t* q = reinterpret_cast<uint32_t*>(const_cast<uint16_t*>(p));
  return uint4{__hip_atomic_load(q, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
               __hip_atomic_load(q + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
               __hip_atomic_load(q + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
               __hip_atomic_load(q + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)};
}

__device__ __forceinline__ void widen_bf16x8(const uint4& r, float (&v)[8]) {
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// The fused combine's part of a down-projection block (bf16 rows), after its
// output stores: count the block's rows in, then combine the tokens whose
// last rows these were.  list: LDS for 1 + (row1 - row0) ints.  Every
// wavefront of the block calls it.
template <int THREADS, int COLS>
__device__ __forceinline__ void fused_combine_tail(const GFuse& F, const GSet& S, int row0, int row1,
                                                   int nblk, int* list) {
  const int tid = threadIdx.x, lane = tid & 63;
  // The block's rows were stored at device scope; once every wavefront's
  // stores have completed they are visible to every XCD, before any counter
  // the block bumps can be seen (so no cache write-back is needed here).
  wait_vm<0>();
  __syncthreads();
  if (tid == 0) list[0] = 0;
  __syncthreads();
  if (tid < 64) {
    for (int r = row0 + lane; r < row1; r += 64) {
      const int t = S.out_token ? S.out_token[r] : r;
      if (t < 0 || t >= F.T) continue;   // not a token row (rows come from the permutation)
      const int old = __hip_atomic_fetch_add(F.cnt + static_cast<int64_t>(t) * F.nb + nblk, 1,
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old == F.expect - 1) list[1 + atomicAdd(&list[0], 1)] = t;
    }
  }
  __syncthreads();
  const int n = list[0];
  constexpr int TPT = COLS / 8;          // threads per owned token, 8 columns each
  constexpr int PASS = THREADS / TPT;    // tokens per pass of the block
  static_assert(COLS % 8 == 0 && THREADS % TPT == 0, "combine split");
  const int64_t Tk = static_cast<int64_t>(F.T) * F.k;
  const uint16_t* o = static_cast<const uint16_t*>(F.o);
  for (int u = tid / TPT; u < n; u += PASS) {
    const int t = list[1 + u];
    const int d = nblk * COLS + (tid % TPT) * 8;
    if (d >= F.D) continue;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // slots in groups of 8: the group's loads first, then the rows in slot order
    for (int j0 = 0; j0 < F.k; j0 += 8) {
      uint4 raw[8];
      int rr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = j0 + e;
        const int r = j < F.k ? F.row_of_slot[static_cast<int64_t>(t) * F.k + j] : -1;
        rr[e] = (r >= 0 && r < Tk) ? r : -1;
        raw[e] = load16_device(o + static_cast<int64_t>(rr[e] < 0 ? 0 : rr[e]) * F.D + d);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (rr[e] < 0) continue;
        float v[8];
        widen_bf16x8(raw[e], v);
        const float wj = F.w[static_cast<int64_t>(t) * F.k + j0 + e];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = __builtin_fmaf(wj, v[i], acc[i]);
      }
    }
    if (F.o_sh) {
      float v[8];
      widen_bf16x8(load16_device(static_cast<const uint16_t*>(F.o_sh) + static_cast<int64_t>(t) * F.D + d), v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    uint32_t wv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      wv[i] = static_cast<uint32_t>(f32_to_bf16(acc[2 * i])) | (static_cast<uint32_t>(f32_to_bf16(acc[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(F.y) + static_cast<int64_t>(t) * F.D + d) =
        uint4{wv[0], wv[1], wv[2], wv[3]};
  }
}

template <class C, bool GATED, int WDT, int ODT>
__global__ __launch_bounds__(C::THREADS, C::WPE) void tiled_gemm_kernel(const GArgs g) {
  constexpr bool FP8 = WDT == DT_FP8;
  constexpr int TF = C::TF, WF = C::WF, S = C::S, P = C::P, BNW = C::BNW;
  constexpr int H = C::H, ROWB = C::ROWB, ROWB8 = C::ROWB8, ROWA = C::ROWA, MF = C::MF;
  constexpr bool A8 = C::A8;
  constexpr int NKS = (MF == 16 || A8) ? 1 : 2;   // MFMAs per fragment pair and sub-step
  // the LDS ring; after the K loop, the staged bf16 output tile (rows padded
  // by 16 bytes)
  constexpr int STAGED = !GATED && ODT == DT_BF16 ? C::BM * (BNW * 2 + 16) : 0;
  constexpr int SMEM = C::LDS > STAGED ? C::LDS : STAGED;
  static_assert(SMEM <= LDS_CU / C::BPC, "LDS per block");
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  // An (empty) statement that names an accumulation register makes the backend
  // select the AGPR form of the MFMAs, so the accumulators live in AGPRs and
  // the VGPRs stay free for fragments.  The sub-channel kernels rescale their
  // accumulators with vector multiplies, so theirs stay in VGPRs (in AGPRs
  // the rescale spilled).
  if constexpr (!C::SUB) asm volatile("" ::: "a0");
  int b = blockIdx.x;
  if constexpr (xcdtile<C>())
    if (xcdtile_ok(g) && !xcdtile_block<C>(g, blockIdx.x, b)) return;
  int si, group, row0, row1, nblk;
  if (!resolve_block(g, b, si, group, row0, row1, nblk)) return;
  // the tile is the same for the whole block: keep it (and everything derived
  // from it, such as the copy base addresses) in scalar registers
  si = __builtin_amdgcn_readfirstlane(si);
  group = __builtin_amdgcn_readfirstlane(group);
  row0 = __builtin_amdgcn_readfirstlane(row0);
  row1 = __builtin_amdgcn_readfirstlane(row1);
  nblk = __builtin_amdgcn_readfirstlane(nblk);
  const GSet& Sg = g.s[si];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Wavefront w runs on SIMD w % 4.  With 8 wavefronts, the two a SIMD hosts
  // get row groups half a tile apart, so the MFMAs a short tile skips (row
  // fragments past its last row) come off every SIMD alike.
  int wm, wn;
  if constexpr (C::WM == 4) {          // 8 wavefronts: 4 row groups x 2 weight groups
    wm = (wave & 1) + 2 * (wave >> 2);
    wn = (wave >> 1) & 1;
  } else {                             // 2 row groups x WN weight groups
    wm = wave / C::WN;
    wn = wave % C::WN;
  }
  // 16x16x32: lane (lr, q) holds row / weight row lr of a fragment and K
  // elements 8q..8q+7 of the sub-step.  32x32x16: lane (l32, hi) holds row
  // l32 and, in MFMA ks of the sub-step, K chunk 2 hi + ks (8 elements each).
  const int lr = lane & (MF - 1), q = lane / MF;
  const int K = Sg.K;
  const int split = Sg.ksplit > 1 ? (b - Sg.block0) % Sg.ksplit : 0;
  const int k_len = Sg.ksplit > 1 ? K / Sg.ksplit : K;
  const int k_beg = split * k_len;
  const int nst = k_len / C::BK;
  const int n_out = Sg.n_out;
  const int n0 = nblk * (GATED ? BNW / 2 : BNW);   // first h column (gated) / output column
  // MF-row fragments of this wavefront that hold tile rows (the rest is padding)
  const int na = min(TF, max(0, (row1 - row0 - wm * TF * MF + MF - 1) / MF));

  // ---- HBM -> LDS copy assignments.  Copy instruction j of a stage fills LDS
  // bytes [1024 j, 1024 j + 1024) of the A or B tile; lane l fills the 16 bytes
  // at 1024 j + 16 l.  Offsets are 32-bit from a wave-uniform base (checked by
  // the launcher).  Rows past the tile and weight rows past n_out are fetched
  // from a valid row instead: they only feed accumulator rows / columns the
  // epilogue never stores, so the copy needs no predication.
  const char* a_base = uniform_ptr(static_cast<const char*>(Sg.a) + static_cast<int64_t>(k_beg) * (A8 ? 1 : 2));
  uint32_t a_off[C::AL];
#pragma unroll
  for (int i = 0; i < C::AL; ++i) {
    const int j = wave * C::AL + i;
    constexpr int LPR = ROWA / 16;                    // lanes per row
    const int tr = (64 / LPR) * j + lane / LPR;
    const int c = upos<ROWA>(tr, lane % LPR);        // logical chunk of this position
    const int r = row0 + tr;
    int64_t arow = 0;
    if (r < row1) {
      arow = Sg.gather ? Sg.gather[r] : r;
      if (static_cast<uint64_t>(arow) >= static_cast<uint64_t>(Sg.a_rows)) arow = 0;  // caller error
    }
    a_off[i] = static_cast<uint32_t>(arow * Sg.lda * (A8 ? 1 : 2) + c * 16);
  }
  // weight bytes of e elements
  auto wbytes = [&](int64_t e) __attribute__((always_inline)) -> int64_t {
    return C::W4 ? e / 2 : FP8 ? e : 2 * e;
  };
  const char* b_base = uniform_ptr(static_cast<const char*>(Sg.w) + wbytes(group * Sg.w_gstride + k_beg));
  uint32_t b_off[C::BL];
#pragma unroll
  for (int i = 0; i < C::BL; ++i) {
    const int j = wave * C::BL + i;
    constexpr int RB = C::ROWBW, LPR = RB / 16;
    const int tr = (64 / LPR) * j + lane / LPR;
    const int c = upos<RB>(tr, lane % LPR);
    int wrow;
    if (GATED) {
      const int n = n0 + (tr & (BNW / 2 - 1));
      wrow = n < n_out ? (tr < BNW / 2 ? 0 : n_out) + n : 0;
    } else {
      wrow = n0 + tr < n_out ? n0 + tr : 0;
    }
    b_off[i] = static_cast<uint32_t>(wbytes(static_cast<int64_t>(wrow) * K) + c * 16);
  }
  // copy instruction k (0..P-1) of stage st: the A instructions, then B
  auto issue_one = [&](int st, int k) __attribute__((always_inline)) {
    char* base = smem + (st % S) * C::STAGE;
    if (k < C::AL) {
      dma16(a_off[k], a_base + st * ROWA, base + (wave * C::AL + k) * 1024);
    } else {
      const int i = k - C::AL;
      dma16(b_off[i], b_base + st * C::ROWBW, base + C::A_BYTES + (wave * C::BL + i) * 1024);
    }
  };
  // MX block scales: wavefront w < NSC copies one part of stage st's scales --
  // the 4 bytes of each of 64 activation rows, or 256 weight rows (4 rows per
  // lane; gate and up rows each contiguous, 4 | n_out).
  [[maybe_unused]] uint32_t sc_off = 0;
  [[maybe_unused]] const char* sc_base = nullptr;
  [[maybe_unused]] int64_t sc_stride = 0;   // bytes between consecutive 128-deep K groups
  if constexpr (C::W4) {
    const int kg0 = k_beg / 128;
    if (wave < C::ASC_I) {
      const int tr = 64 * wave + lane;
      const int r = row0 + tr;
      int64_t arow = 0;
      if (r < row1) {
        arow = Sg.gather ? Sg.gather[r] : r;
        if (static_cast<uint64_t>(arow) >= static_cast<uint64_t>(Sg.a_rows)) arow = 0;
      }
      sc_off = static_cast<uint32_t>(arow * 4);
      sc_stride = static_cast<int64_t>(Sg.a_mx_rows) * 4;
      sc_base = uniform_ptr(reinterpret_cast<const char*>(Sg.a_mx) + kg0 * sc_stride);
    } else if (wave < C::NSC) {
      const int tr = 256 * (wave - C::ASC_I) + 4 * lane;   // first of the lane's 4 tile rows
      int wrow;
      if (GATED) {
        const int n = n0 + (tr & (BNW / 2 - 1));
        wrow = n < n_out ? (tr < BNW / 2 ? 0 : n_out) + n : 0;
      } else {
        wrow = n0 + tr < n_out ? n0 + tr : 0;
      }
      sc_off = static_cast<uint32_t>(wrow * 4);
      sc_stride = static_cast<int64_t>(Sg.NB) * 4;
      sc_base = uniform_ptr(reinterpret_cast<const char*>(Sg.w_mx) + group * Sg.w_mx_gstride + kg0 * sc_stride);
    }
  }
  if constexpr (C::SUB) {
    // wavefront w < ASC_I copies the scales of tile rows [64 w, 64 w + 64)
    // for the stage's slice ([slice][row] fp32, gathered rows)
    if (wave < C::ASC_I) {
      const int r = row0 + 64 * wave + lane;
      int64_t arow = 0;
      if (r < row1) {
        arow = Sg.gather ? Sg.gather[r] : r;
        if (static_cast<uint64_t>(arow) >= static_cast<uint64_t>(Sg.a_rows)) arow = 0;
      }
      sc_off = static_cast<uint32_t>(arow * 4);
      sc_stride = static_cast<int64_t>(Sg.a_sub_rows) * 4;
      sc_base = uniform_ptr(reinterpret_cast<const char*>(Sg.a_sub) + (k_beg / kSubChannel) * sc_stride);
    }
  }
  auto issue_scales = [&](int st) __attribute__((always_inline)) {
    char* sc_lds = smem + (st % S) * C::STAGE + C::A_BYTES + C::B_BYTES;
    if constexpr (C::W4) {
      if (wave < C::ASC_I)
        dma4(sc_off, sc_base + st * sc_stride, sc_lds + wave * 256);
      else if (wave < C::NSC)
        dma16(sc_off, sc_base + st * sc_stride, sc_lds + C::ASC_BYTES + (wave - C::ASC_I) * 1024);
    } else if constexpr (C::SUB) {
      if (wave < C::ASC_I) dma4(sc_off, sc_base + (st / (kSubChannel / C::BK)) * sc_stride, sc_lds + wave * 256);
    }
  };
  // Waits for copies: this wavefront issues P copies per stage, plus one scale
  // copy if it is a scale copier.
  auto wait_stages = [&](int newer, auto m) __attribute__((always_inline)) {
    constexpr int M = decltype(m)::value;
    if constexpr (C::W4 || C::SUB) {
      if (wave < C::NSC) wait_newer<P + 1, M>(newer);
      else wait_newer<P, M>(newer);
    } else {
      wait_newer<P, M>(newer);
    }
  };

  // acc[f][i]: weight fragment f (MF weight rows) x row fragment i (MF rows)
  using AccT = typename std::conditional<MF == 16, f32x4, f32x16>::type;
  AccT acc[WF][TF];
#pragma unroll
  for (int f = 0; f < WF; ++f)
#pragma unroll
    for (int i = 0; i < TF; ++i)
#pragma unroll
      for (int e = 0; e < MF * MF / 64; ++e) acc[f][i][e] = 0.f;

  // weight tile row of fragment f of this wavefront
  auto wrow_of = [&](int f) __attribute__((always_inline)) -> int {
    constexpr int HC = BNW / 2 / C::WN;   // h columns per wavefront (gated)
    return GATED ? ((f < WF / 2 ? 0 : BNW / 2) + wn * HC + (f % (WF / 2)) * MF + lr)
                 : (wn * WF * MF + f * MF + lr);
  };
  // a[i][ks]; b[f][ks] (bf16) or b[f][0] (fp8: the lane's weight bytes of the
  // sub-step, 8 or 16); w[f][ks]: fp8 weights decoded
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  using B8 = typename std::conditional<MF == 16, u32x2, u32x4>::type;
  using BT = typename std::conditional<FP8, B8, bf16x8>::type;
  struct FragW {     // bf16 activations
    bf16x8 a[TF][NKS];
    BT b[WF][FP8 ? 1 : NKS];
    bf16x8 w[FP8 ? WF : 1][NKS];
  };
  struct Frag8 {     // fp8 activations and weights: a lane's 32 bytes of a sub-step
    i32x8 a[TF];
    i32x8 b[WF];
  };
  struct Frag4 {     // MXFP8 activations, MXFP4 weights, and the lane's block scales
    i32x8 a[TF];
    u32x4 b[WF];
    int sa[TF];
    int sb[WF];
  };
  struct Frag8S {    // fp8 activations with their rows' slice scales s = m 2^(e - 127)
    i32x8 a[TF];
    i32x8 b[WF];
    float s[TF];
    int e[TF];
    float m[TF];
  };
  using Frag = typename std::conditional<
      C::W4, Frag4,
      typename std::conditional<A8, typename std::conditional<C::SUB, Frag8S, Frag8>::type, FragW>::type>::type;
  // 16-byte chunk (of the tile row) holding the lane's K elements of sub-step
  // h of a stage, in MFMA ks
  auto chunk_of = [&](int h, int ks) __attribute__((always_inline)) -> int {
    return MF == 16 ? 4 * h + q : 4 * h + 2 * q + ks;
  };
  // fragments of sub-step t (K elements [32 t, 32 t + 32) of the tile)
  // fp8 x fp8 (32x32x64): lane (lr, q) takes bytes [64 h + 32 q, + 32) of its
  // row in sub-step h, two 16-byte chunks, for either operand
  auto readf = [&](Frag& F, int t) __attribute__((always_inline)) {
    const int h = t % H;
    const char* base = smem + ((t / H) % S) * C::STAGE;
    const char* bb = base + C::A_BYTES;
    if constexpr (C::W4) {
      // MX operands follow the matrix unit's own K order, so that its two
      // 32-element scale blocks of sub-step h are the tile's blocks 2h, 2h + 1:
      // lane group q takes fp8 K elements [16 q, +16) and [32 + 16 q, +16) of
      // the sub-step (chunks 4h + q, 4h + 2 + q) and fp4 elements [32 q, +32)
      // (16 bytes: chunk 2h + q of the weight row), and the scales of block
      // 2h + q of its activation row and of its weight row
      const char* asc = bb + C::B_BYTES;
      const char* bsc = asc + C::ASC_BYTES;
#pragma unroll
      for (int i = 0; i < TF; ++i) {
        const int r = wm * TF * MF + MF * i + lr;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(base + r * ROWB8 + upos<ROWB8>(r, 4 * h + q) * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(base + r * ROWB8 + upos<ROWB8>(r, 4 * h + 2 + q) * 16);
        F.a[i] = i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                       static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                       static_cast<int>(hi[2]), static_cast<int>(hi[3])};
        F.sa[i] = *reinterpret_cast<const uint8_t*>(asc + 4 * r + 2 * h + q);
      }
#pragma unroll
      for (int f = 0; f < WF; ++f) {
        constexpr int RB = C::ROWBW;
        const int tr = wrow_of(f);
        F.b[f] = *reinterpret_cast<const u32x4*>(bb + tr * RB + upos<RB>(tr, 2 * h + q) * 16);
        F.sb[f] = *reinterpret_cast<const uint8_t*>(bsc + 4 * tr + 2 * h + q);
      }
      return;
    } else if constexpr (A8) {
      auto rd = [&](const char* tile, int row) __attribute__((always_inline)) -> i32x8 {
        const int c0 = 4 * h + 2 * q;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(tile + row * ROWB8 + upos<ROWB8>(row, c0) * 16);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(tile + row * ROWB8 + upos<ROWB8>(row, c0 + 1) * 16);
        return i32x8{static_cast<int>(lo[0]), static_cast<int>(lo[1]), static_cast<int>(lo[2]),
                     static_cast<int>(lo[3]), static_cast<int>(hi[0]), static_cast<int>(hi[1]),
                     static_cast<int>(hi[2]), static_cast<int>(hi[3])};
      };
#pragma unroll
      for (int i = 0; i < TF; ++i) F.a[i] = rd(base, wm * TF * MF + MF * i + lr);
#pragma unroll
      for (int f = 0; f < WF; ++f) F.b[f] = rd(bb, wrow_of(f));
      if constexpr (C::SUB) {
        const char* asc = bb + C::B_BYTES;
#pragma unroll
        for (int i = 0; i < TF; ++i)
          F.s[i] = *reinterpret_cast<const float*>(asc + 4 * (wm * TF * MF + MF * i + lr));
      }
      return;
    } else {
#pragma unroll
    for (int i = 0; i < TF; ++i) {
      const int r = wm * TF * MF + MF * i + lr;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        F.a[i][ks] = *reinterpret_cast<const bf16x8*>(base + r * ROWB + upos<ROWB>(r, chunk_of(h, ks)) * 16);
    }
#pragma unroll
    for (int f = 0; f < WF; ++f) {
      const int tr = wrow_of(f);
      if constexpr (FP8) {
        if constexpr (MF == 16)
          F.b[f][0] = *reinterpret_cast<const B8*>(bb + tr * ROWB8 + upos<ROWB8>(tr, 2 * h + (q >> 1)) * 16 +
                                                   (q & 1) * 8);
        else
          F.b[f][0] = *reinterpret_cast<const B8*>(bb + tr * ROWB8 + upos<ROWB8>(tr, 2 * h + q) * 16);
      } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          F.b[f][ks] = *reinterpret_cast<const bf16x8*>(bb + tr * ROWB + upos<ROWB>(tr, chunk_of(h, ks)) * 16);
      }
    }
    }
  };
  // Use the fragments in an empty statement so that the compiler's own wait
  // for them lands here (before the barrier) and not in front of the MFMAs.
  auto settle = [&](Frag& F) __attribute__((always_inline)) {
    if constexpr (C::W4) {
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
      for (int i = 0; i < TF; ++i) asm volatile("" ::"v"(F.a[i]), "v"(F.sa[i]));
#pragma unroll
      for (int f = 0; f < WF; ++f) asm volatile("" ::"v"(F.b[f]), "v"(F.sb[f]));
#endif
      return;
    } else if constexpr (A8) {
      // (a 32-byte "v" operand is not valid for the host target: device pass only)
#if defined(__HIP_DEVICE_COMPILE__)
#pragma unroll
      for (int i = 0; i < TF; ++i) asm volatile("" ::"v"(F.a[i]));
#pragma unroll
      for (int f = 0; f < WF; ++f) asm volatile("" ::"v"(F.b[f]));
#endif
      if constexpr (C::SUB) {
#pragma unroll
        for (int i = 0; i < TF; ++i) F.m[i] = split_scale(F.s[i], F.e[i]);
      }
      return;
    } else {
#pragma unroll
    for (int i = 0; i < TF; ++i)
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) asm volatile("" ::"v"(F.a[i][ks]));
#pragma unroll
    for (int f = 0; f < WF; ++f)
#pragma unroll
      for (int ks = 0; ks < (FP8 ? 1 : NKS); ++ks) asm volatile("" ::"v"(F.b[f][ks]));
    if constexpr (FP8) {
#pragma unroll
      for (int f = 0; f < WF; ++f) {
        F.w[f][0] = fp8x8_to_bf16x8(F.b[f][0][0], F.b[f][0][1]);
        if constexpr (MF == 32) F.w[f][1] = fp8x8_to_bf16x8(F.b[f][0][2], F.b[f][0][3]);
      }
    }
    }
  };
  // Sub-channel scales (the "Qwen 3.5 MoE on Ironwood" page, MoE track, GMM
  // v2: fp8 activations with one scale per 512-element slice).  A row's sum
  // is sum_j s_j P_j over its slices j, s_j = m_j 2^e_j.  The matrix cores
  // apply 2^e_j as the activation block scale; the accumulators hold the sum
  // in units of the current slice's mantissa, so at each slice's first
  // sub-step they are multiplied by m_(j-1) / m_j (between 1/2 and 2: no
  // overflow, one rounding), and the epilogue multiplies by the last m.
  [[maybe_unused]] float mprev[C::SUB ? TF : 1];
  auto rescale = [&](const Frag& F, int t) __attribute__((always_inline)) {
    if constexpr (C::SUB) {
      constexpr int SPS = kSubChannel / C::KSUB;   // sub-steps per slice
      if (t % SPS == 0) {
        if (t > 0) {
#pragma unroll
          for (int i = 0; i < TF; ++i) {
            const float r = mprev[i] / F.m[i];
#pragma unroll
            for (int f = 0; f < WF; ++f)
#pragma unroll
              for (int e = 0; e < MF * MF / 64; ++e) acc[f][i][e] *= r;
          }
        }
#pragma unroll
        for (int i = 0; i < TF; ++i) mprev[i] = F.m[i];
      }
    }
  };
  // MFMAs of one sub-step, row fragment by row fragment; fragments past the
  // tile's last row (i >= na, a uniform branch) are skipped.
  auto mma = [&](const Frag& F) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TF; ++i) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        if (i < na) {
#pragma unroll
          for (int f = 0; f < WF; ++f) {
            if constexpr (C::W4) {
              // e2m1 weights (format code 4, the low four dwords) x e4m3
              // activations (code 0), each with its E8M0 block scale
              const u32x4& w = F.b[f];
              const i32x8 w8{static_cast<int>(w[0]), static_cast<int>(w[1]), static_cast<int>(w[2]),
                             static_cast<int>(w[3]), 0, 0, 0, 0};
              acc[f][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w8, F.a[i], acc[f][i], 4, 0, 0,
                                                                          F.sb[f], 0, F.sa[i]);
            } else if constexpr (C::SUB) {
              // e4m3 x e4m3, the activation rows' slice scales' powers of two
              // as their block scales (the mantissas are applied outside)
              acc[f][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.b[f], F.a[i], acc[f][i], 0, 0,
                                                                          0, 127, 0, F.e[i]);
            } else if constexpr (A8) {
              // e4m3 x e4m3 (format codes 0), unit block scales (exponent 127)
              acc[f][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.b[f], F.a[i], acc[f][i], 0, 0,
                                                                          0, 127, 0, 127);
            } else {
              bf16x8 w;
              if constexpr (FP8) w = F.w[f][ks];
              else w = F.b[f][ks];
              if constexpr (MF == 16)
                acc[f][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w, F.a[i][ks], acc[f][i], 0, 0, 0);
              else
                acc[f][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(w, F.a[i][ks], acc[f][i], 0, 0, 0);
            }
          }
        }
      }
    }
  };
  // copies [c P1, (c + 1) P1) of a stage: chunk c of its H chunks
  constexpr int P1 = C::P1;
  auto chunk_lo = [](auto c) { return std::integral_constant<int, (decltype(c)::value * P1 < P ? decltype(c)::value * P1 : P)>(); };
  auto chunk_hi = [](auto c) { return std::integral_constant<int, ((decltype(c)::value + 1) * P1 < P ? (decltype(c)::value + 1) * P1 : P)>(); };
  // Sub-step t, phase PH = t % H within its stage.  When sub-step t + 1 opens
  // a stage (PH == H - 1), that stage has landed (own copies; everyone's after
  // the barrier, which also frees the slot of the stage just finished for the
  // stage S further on).  That stage's copies go out in H chunks: the first
  // in this sub-step, the others in the next stage's first H - 1 sub-steps.
  // A sub-step issues its chunk of copies first, then reads sub-step t + 1's
  // fragments, then runs t's MFMAs: copies issued ahead of the LDS reads and
  // MFMAs measured about 5% faster than copies spread among the MFMAs.
  auto issue_chunk = [&](int st, auto c) __attribute__((always_inline)) {
#pragma unroll
    for (int k = decltype(chunk_lo(c))::value; k < decltype(chunk_hi(c))::value; ++k) issue_one(st, k);
  };
  auto step = [&](Frag& cur, Frag& nxt, int t, auto ph) __attribute__((always_inline)) {
    constexpr int PH = decltype(ph)::value;
    if constexpr (PH == H - 1) {
      const int x = (t + 1) / H - 1;   // the stage finished by this sub-step
      wait_stages(max(0, min(S - 2, nst - 2 - x)), std::integral_constant<int, S - 2>());
      settle(cur);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (x + S < nst) {
        issue_scales(x + S);
        issue_chunk(x + S, std::integral_constant<int, 0>());
      }
      readf(nxt, t + 1);   // t + 1 == nst * H reads a stale slot that is never used
      rescale(cur, t);
      mma(cur);
    } else {
      const int x = t / H - 1;         // its slot was freed by the last barrier
      settle(cur);                     // (decodes fp8 weights)
      if (x >= 0 && x + S < nst) issue_chunk(x + S, std::integral_constant<int, PH + 1>());
      readf(nxt, t + 1);
      rescale(cur, t);
      mma(cur);
    }
  };

  // ---- prologue: S stages in flight, stage 0's fragments read
#pragma unroll
  for (int st = 0; st < S; ++st)
    if (st < nst) {
      issue_scales(st);
#pragma unroll
      for (int k = 0; k < P; ++k) issue_one(st, k);
    }
  Frag F0, F1;
  wait_stages(min(S - 1, nst - 1), std::integral_constant<int, S - 1>());
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  readf(F0, 0);
  // nst * H sub-steps, a multiple of 2 and of H (with one sub-step per stage,
  // nst is even: checked by the launcher); one loop trip covers UNR of them,
  // each with its phase known at compile time
  constexpr int UNR = H > 2 ? H : 2;
  auto sub = [&](int t, auto ic) __attribute__((always_inline)) {   // sub-step t + I of a trip
    constexpr int I = decltype(ic)::value;
    if constexpr (I % 2 == 0) step(F0, F1, t + I, std::integral_constant<int, I % H>());
    else step(F1, F0, t + I, std::integral_constant<int, I % H>());
  };
  for (int t = 0; t < nst * H; t += UNR) {
    sub(t, std::integral_constant<int, 0>());
    sub(t, std::integral_constant<int, 1>());
    if constexpr (UNR >= 4) {
      sub(t, std::integral_constant<int, 2>());
      sub(t, std::integral_constant<int, 3>());
    }
    if constexpr (UNR >= 8) {
      sub(t, std::integral_constant<int, 4>());
      sub(t, std::integral_constant<int, 5>());
      sub(t, std::integral_constant<int, 6>());
      sub(t, std::integral_constant<int, 7>());
    }
  }
  wait_vm<0>();   // no copy may still be in flight when the block retires

  // ---- epilogue.  16x16: lane (lr, q) holds C[row lr of fragment i][columns
  // 4q..4q+3 of fragment f].  32x32: accumulator element 4g + j of lane
  // (lr, q) holds C[row lr][column 8g + 4q + j].  Each group of 4 columns is
  // stored together (8 bytes in bf16, 16 in fp32); column groups outermost, so
  // each group's scales are loaded once.  Plain bf16 tiles (the down
  // projection) are staged in the LDS (free once the K loop is done) and then
  // written row by row, 16 bytes per lane: a lane's own 8-byte pieces reach
  // HBM as partial lines (the Ling prefill down projection wrote 4.07 GB for
  // its 2.42 GB of rows; staged: 5.16 -> 4.79 ms).  The gated tiles' rows are
  // half as wide and the staging measured 1 % slower there.  The staged rows
  // are stored with the non-temporal hint, keeping the cache for the weight
  // slabs the tiles share (Qwen prefill down projection 1.53 -> 1.46 ms, Ling
  // decode 0.80 -> 0.79 ms, Ling prefill and Gemma level).
  const float* sc = Sg.scale ? Sg.scale + group * Sg.s_gstride : nullptr;
  constexpr int OCOLS = GATED ? BNW / 2 / C::WN : BNW / C::WN;   // output columns per wavefront
  constexpr int NG = MF == 16 ? 1 : MF / 8;                      // column groups per fragment and lane
  constexpr int TCOLS = GATED ? BNW / 2 : BNW;                   // output columns of the block
  constexpr int SROW = TCOLS * 2 + 16;                           // LDS bytes per staged row (padded)
  const int col_w = n0 + wn * OCOLS;
  char* outb = static_cast<char*>(Sg.out) + split * Sg.split_stride * (ODT == DT_F32 ? 4 : 2);
  const bool fuse = g.fc.cnt != nullptr;   // fused combine (ungated bf16 launches only)
  const bool stage_out = !GATED && ODT == DT_BF16 && !fuse;
  if constexpr (!GATED && ODT == DT_BF16) {
    static_assert(SMEM >= C::BM * SROW, "staged output tile");
    if (stage_out) __syncthreads();   // every wavefront is done with the LDS ring
  }
#pragma unroll
  for (int fg = 0; fg < (GATED ? WF / 2 : WF) * NG; ++fg) {
    const int f = fg / NG, g = fg % NG;
    const int col = col_w + f * MF + (MF == 16 ? 4 * q : 8 * g + 4 * q);   // first of the lane's 4 columns
    const bool col_ok = col < n_out;                                       // n_out is a multiple of 4
    float s0[4], s1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      s0[j] = (sc && col_ok) ? sc[col + j] : 1.f;
      s1[j] = (GATED && sc && col_ok) ? sc[n_out + col + j] : 1.f;
    }
#pragma unroll
    for (int i = 0; i < TF; ++i) {
      const int r = row0 + wm * TF * MF + i * MF + lr;
      if (r >= row1 || !col_ok) continue;
      float ra = 1.f;   // the row's activation scale (fp8 activations)
      if constexpr (A8 && !C::W4) ra = Sg.a_scale[Sg.gather ? Sg.gather[r] : r];
      if constexpr (C::SUB) {
        int e_unused;
        ra = split_scale(ra, e_unused);   // the last slice's mantissa (its power of two is in the sums)
      }
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = 4 * g + j;
        if constexpr (GATED)
          v[j] = act_fn(Sg.act, acc[f][i][e] * ra * s0[j]) * (acc[f + WF / 2][i][e] * ra * s1[j]);
        else
          v[j] = acc[f][i][e] * ra * s0[j];
      }
      const int64_t o = static_cast<int64_t>(r) * Sg.ldo + col;
      if constexpr (ODT == DT_BF16) {
        const uint32_t p0 = static_cast<uint32_t>(f32_to_bf16(v[0])) | (static_cast<uint32_t>(f32_to_bf16(v[1])) << 16);
        const uint32_t p1 = static_cast<uint32_t>(f32_to_bf16(v[2])) | (static_cast<uint32_t>(f32_to_bf16(v[3])) << 16);
        if (GATED) {
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(outb) + o) = uint2{p0, p1};
        } else if (stage_out) {
          *reinterpret_cast<uint2*>(smem + (r - row0) * SROW + (col - n0) * 2) = uint2{p0, p1};
        } else {
          // rows the fused combine reads on other XCDs: device-scope stores,
          // written through this XCD's cache
          uint32_t* q = reinterpret_cast<uint32_t*>(reinterpret_cast<uint16_t*>(outb) + o);
          __hip_atomic_store(q, p0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(q + 1, p1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(outb) + o) = float4{v[0], v[1], v[2], v[3]};
      }
    }
  }
  if constexpr (!GATED && ODT == DT_BF16) {
    if (stage_out) {
      // the staged tile, rows [row0, row1) x columns [n0, n0 + TCOLS) within
      // n_out (a multiple of 4: 8-byte pieces at the row's end), 16 bytes a lane
      __syncthreads();
      constexpr int CPR = TCOLS / 8;   // 16-byte chunks per row
      const int nrows = row1 - row0, ncols = min(TCOLS, n_out - n0);
      for (int idx = threadIdx.x; idx < nrows * CPR; idx += C::THREADS) {
        const int rr = idx / CPR, c8 = (idx % CPR) * 8;
        if (c8 >= ncols) continue;
        const char* src = smem + rr * SROW + c8 * 2;
        uint16_t* dst = reinterpret_cast<uint16_t*>(outb) + static_cast<int64_t>(row0 + rr) * Sg.ldo + n0 + c8;
        if (c8 + 8 <= ncols)   // streaming stores: the rows are read once, by the combine
          __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(src), reinterpret_cast<u32x4*>(dst));
        else
          *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
      }
    }
  }
  if constexpr (!GATED && ODT == DT_BF16) {
    static_assert(C::LDS >= 4 * (C::BM + 1), "combine list");
    if (g.fc.cnt) fused_combine_tail<C::THREADS, BNW>(g.fc, Sg, row0, row1, nblk, reinterpret_cast<int*>(smem));
  }
}

template <class C, bool GATED, int WDT, int ODT>
hipError_t launch_one(const GArgs& g, hipStream_t s) {
  int grid = g.total_blocks;
  if constexpr (xcdtile<C>())
    if (xcdtile_ok(g)) grid = xcdtile_grid<C>(g);
  tiled_gemm_kernel<C, GATED, WDT, ODT><<<grid, C::THREADS, 0, s>>>(g);
  return hipGetLastError();
}

template <int BM, int BNW, int WM, int WN, int BPC, int MF>
hipError_t dispatch(const GArgs& g, bool gated, int w_dtype, int out_dtype, int a_dtype, hipStream_t s) {
  using CB = Cfg<BM, BNW, WM, WN, BPC, false, 32, MF>;
  // fp8 weights 64 deep where three such stages fit in the block's LDS share
  constexpr bool W1 = BM == 128 && BNW == 512;
  using C8 = Cfg<BM, BNW, (W1 ? 1 : WM), (W1 ? 8 : WN), BPC, true, (BPC == 1 ? 64 : 32), MF>;
  if (a_dtype == DT_MXFP8) {
    // MXFP8 x MXFP4: one block per CU, scaled 32x32x64 MFMAs, 128-deep stages
    if constexpr (BPC == 1) {
      using CW = Cfg<BM, BNW, WM, WN, 1, true, 128, 32, true, true>;
      if (w_dtype != DT_MXFP4 || out_dtype != DT_BF16) return hipErrorInvalidValue;
      return gated ? launch_one<CW, true, DT_MXFP4, DT_BF16>(g, s) : launch_one<CW, false, DT_MXFP4, DT_BF16>(g, s);
    }
    return hipErrorInvalidValue;
  }
  if (a_dtype == DT_FP8) {
    // fp8 x fp8: one block per CU, 32x32x64 MFMAs
    if constexpr (BPC == 1) {
      using CA = Cfg<BM, BNW, WM, WN, 1, true, BK8A, 32, true>;
      if (w_dtype != DT_FP8 || out_dtype != DT_BF16) return hipErrorInvalidValue;
      return gated ? launch_one<CA, true, DT_FP8, DT_BF16>(g, s) : launch_one<CA, false, DT_FP8, DT_BF16>(g, s);
    }
    return hipErrorInvalidValue;
  }
  if (a_dtype == DT_FP8S) {
    // fp8 x fp8 with sub-channel activation scales: 256-row tiles only (the
    // 128 x 512 block's registers do not hold the rescaled accumulators),
    // 128-deep stages in two slots with the stage's scale row (measured 8 %
    // faster than 64-deep ones in four)
    if constexpr (BPC == 1 && BM == 256) {
      using CS = Cfg<BM, BNW, WM, WN, 1, true, 128, 32, true, false, true>;
      if (w_dtype != DT_FP8 || out_dtype != DT_BF16) return hipErrorInvalidValue;
      return gated ? launch_one<CS, true, DT_FP8, DT_BF16>(g, s) : launch_one<CS, false, DT_FP8, DT_BF16>(g, s);
    }
    return hipErrorInvalidValue;
  }
  if (gated) {
    if (w_dtype == DT_BF16 && out_dtype == DT_BF16) return launch_one<CB, true, DT_BF16, DT_BF16>(g, s);
    if (w_dtype == DT_FP8 && out_dtype == DT_BF16) return launch_one<C8, true, DT_FP8, DT_BF16>(g, s);
  } else {
    if (w_dtype == DT_BF16 && out_dtype == DT_BF16) return launch_one<CB, false, DT_BF16, DT_BF16>(g, s);
    if (w_dtype == DT_FP8 && out_dtype == DT_BF16) return launch_one<C8, false, DT_FP8, DT_BF16>(g, s);
    if (w_dtype == DT_BF16 && out_dtype == DT_F32) return launch_one<CB, false, DT_BF16, DT_F32>(g, s);
  }
  return hipErrorInvalidValue;
}

// Decode-sized groups: 32 rows x 128 weight rows, four wavefronts of 32 rows
// x 32 weight rows, two blocks per CU, 128-deep stages (128-byte fp8 or
// 256-byte bf16 weight-row requests, four MFMA sub-steps per stage) in a ring
// of two or three.  The weights stream through the LDS ring, so a block keeps
// its next stage in flight without holding it in registers.  bf16 weights
// over a long K (at least kSmallDeepK) take 256-deep stages instead, one
// block per CU (512-byte weight-row requests; measured on the Qwen decode
// gate/up projection 1067 -> 1035 us; a short K keeps 128-deep stages).
constexpr int kSmallBNW = 128;
constexpr int kSmallBK = 128;
constexpr int kSmallDeepK = 2048;
hipError_t dispatch_small(const GArgs& g, bool gated, int w_dtype, int out_dtype, int a_dtype,
                          hipStream_t s) {
  using C = Cfg<32, kSmallBNW, 1, 4, 2, true, kSmallBK, 16>;
  using CB = Cfg<32, kSmallBNW, 1, 4, 2, false, kSmallBK, 16>;
  using CBD = Cfg<32, kSmallBNW, 1, 4, 1, false, 256, 16>;
  bool deep = w_dtype == DT_BF16;
  for (int i = 0; i < g.nsets; ++i) {
    const int k = g.s[i].K / (g.s[i].ksplit > 1 ? g.s[i].ksplit : 1);
    if (k % C::BK) return hipErrorInvalidValue;
    deep = deep && k % CBD::BK == 0 && k >= kSmallDeepK;
  }
  if (a_dtype != DT_BF16 || out_dtype != DT_BF16) return hipErrorInvalidValue;
  if (w_dtype == DT_FP8)
    return gated ? launch_one<C, true, DT_FP8, DT_BF16>(g, s) : launch_one<C, false, DT_FP8, DT_BF16>(g, s);
  if (w_dtype == DT_BF16 && deep)
    return gated ? launch_one<CBD, true, DT_BF16, DT_BF16>(g, s) : launch_one<CBD, false, DT_BF16, DT_BF16>(g, s);
  if (w_dtype == DT_BF16)
    return gated ? launch_one<CB, true, DT_BF16, DT_BF16>(g, s) : launch_one<CB, false, DT_BF16, DT_BF16>(g, s);
  return hipErrorInvalidValue;
}

// The down projection of decode-sized groups with bf16 weights: 32 rows x 64
// weight rows, four wavefronts of 32 x 16, twice the blocks of the 32 x 128
// shape on the same M-tile table; stages as there (256 deep, one block per CU,
// from kSmallDeepK).  Measured on the Qwen decode down projection (K = 1024)
// 0.501 -> 0.487 ms.  With fp8 weights the same shape was slower (Ling decode
// down projection 0.80 -> 0.93 ms with 128-deep stages, 1.01 ms with 256-deep
// ones), so fp8 weights keep the 32 x 128 shape.
hipError_t dispatch_small_down(const GArgs& g, bool gated, int w_dtype, int out_dtype, int a_dtype,
                               hipStream_t s) {
  using CB = Cfg<32, 64, 1, 4, 2, false, kSmallBK, 16>;
  using CBD = Cfg<32, 64, 1, 4, 1, false, 256, 16>;
  bool deep = true;
  for (int i = 0; i < g.nsets; ++i) {
    const int k = g.s[i].K / (g.s[i].ksplit > 1 ? g.s[i].ksplit : 1);
    if (k % CB::BK) return hipErrorInvalidValue;
    deep = deep && k % CBD::BK == 0 && k >= kSmallDeepK;
  }
  if (gated || w_dtype != DT_BF16 || a_dtype != DT_BF16 || out_dtype != DT_BF16) return hipErrorInvalidValue;
  return deep ? launch_one<CBD, false, DT_BF16, DT_BF16>(g, s) : launch_one<CB, false, DT_BF16, DT_BF16>(g, s);
}

// Decode-sized groups with quantised activations: 64 rows x 256 weight rows,
// four wavefronts of 64 x 64 (one 32 x 32 fragment pair of gate and up rows
// each), two blocks per CU, 128-deep stages; fp8 x fp8, or MXFP8 x MXFP4 with
// the block-scale tiles.
hipError_t dispatch_smallq(const GArgs& g, bool gated, int w_dtype, int out_dtype, int a_dtype,
                           hipStream_t s) {
  using CA = Cfg<64, 256, 1, 4, 2, true, 128, 32, true>;
  using CW = Cfg<64, 256, 1, 4, 2, true, 128, 32, true, true>;
  using CS = Cfg<64, 256, 1, 4, 2, true, 64, 32, true, false, true>;   // 64 deep: the scales fit the LDS share
  if (out_dtype != DT_BF16) return hipErrorInvalidValue;
  if (a_dtype == DT_FP8 && w_dtype == DT_FP8)
    return gated ? launch_one<CA, true, DT_FP8, DT_BF16>(g, s) : launch_one<CA, false, DT_FP8, DT_BF16>(g, s);
  if (a_dtype == DT_FP8S && w_dtype == DT_FP8)
    return gated ? launch_one<CS, true, DT_FP8, DT_BF16>(g, s) : launch_one<CS, false, DT_FP8, DT_BF16>(g, s);
  if (a_dtype == DT_MXFP8 && w_dtype == DT_MXFP4)
    return gated ? launch_one<CW, true, DT_MXFP4, DT_BF16>(g, s) : launch_one<CW, false, DT_MXFP4, DT_BF16>(g, s);
  return hipErrorInvalidValue;
}

// weight rows per block of a shape
int block_width(int shape) {
  return shape == TILED_WIDE ? 512 : shape == TILED_SMALL ? kSmallBNW : shape == TILED_SMALLD ? 64 : 256;
}

}  // namespace

int tiled_bm(int shape) {
  return shape == TILED_TALL ? 256 : (shape == TILED_SMALL || shape == TILED_SMALLD) ? 32
         : shape == TILED_SMALLQ ? 64 : 128;
}

int tiled_k_multiple() { return 2 * KS; }

// fp8 x fp8: K a multiple of the 128-deep stage (or of two 64-deep ones)
int tiled_k_multiple_a8() { return 128; }

int tiled_k_multiple_small() { return kSmallBK; }

int tiled_blocks_n(int shape, bool gated, int n_out) {
  const int w = gated ? block_width(shape) / 2 : block_width(shape);
  return (n_out + w - 1) / w;
}

bool tiled_offsets_fit(int64_t a_rows, int64_t lda, int64_t w_rows, int64_t K, int w_dtype) {
  const int64_t w_bytes = w_dtype == DT_MXFP4 ? w_rows * K / 2 : w_rows * K * (w_dtype == DT_FP8 ? 1 : 2);
  return a_rows * lda * 2 < (int64_t(1) << 32) && w_bytes < (int64_t(1) << 32);
}

hipError_t launch_tiled_gemm(const GArgs& g, int shape, bool gated, int w_dtype, int out_dtype,
                             int a_dtype, hipStream_t s) {
  if (g.total_blocks <= 0) return hipSuccess;
  for (int i = 0; i < g.nsets; ++i) {
    const GSet& S = g.s[i];
    const int ks = S.ksplit > 1 ? S.ksplit : 1;
    if ((S.K / ks) % (2 * KS) || S.bm != tiled_bm(shape) || S.n_out % 4) return hipErrorInvalidValue;
    if (a_dtype == DT_FP8 && ((S.K / ks) % tiled_k_multiple_a8() || !S.a_scale)) return hipErrorInvalidValue;
    if (a_dtype == DT_FP8S && (ks != 1 || S.K % kSubChannel || !S.a_scale || !S.a_sub || S.a_sub_rows < S.a_rows))
      return hipErrorInvalidValue;
    if (a_dtype == DT_MXFP8 && ((S.K / ks) % tiled_k_multiple_a8() || !S.a_mx || !S.w_mx ||
                                S.a_mx_rows < S.a_rows || S.NB % 4))
      return hipErrorInvalidValue;
    if (!tiled_offsets_fit(S.a_rows, S.lda, S.NB, S.K, w_dtype)) return hipErrorInvalidValue;
  }
  switch (shape) {
    case TILED_TALL: return dispatch<256, 256, 4, 2, 1, 16>(g, gated, w_dtype, out_dtype, a_dtype, s);
    case TILED_WIDE: return dispatch<128, 512, 2, 4, 1, 16>(g, gated, w_dtype, out_dtype, a_dtype, s);
    case TILED_NARROW: return dispatch<128, 256, 2, 2, 2, 16>(g, gated, w_dtype, out_dtype, a_dtype, s);
    case TILED_SMALL: return dispatch_small(g, gated, w_dtype, out_dtype, a_dtype, s);
    case TILED_SMALLQ: return dispatch_smallq(g, gated, w_dtype, out_dtype, a_dtype, s);
    case TILED_SMALLD: return dispatch_small_down(g, gated, w_dtype, out_dtype, a_dtype, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace moe
