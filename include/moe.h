/*
 * moe.h -- C ABI of the MI355X (gfx950) routed Mixture-of-Experts FFN layer.
 *
 * The layer is  y = Router(x) + SharedExpert(x)  ("Qwen 3.5 MoE on Ironwood"
 * page, model-architecture section): fp32 router logits, top-k softmax with
 * renormalisation, a stable permutation of the (token, slot) assignments by
 * expert, a grouped gated expert FFN (gate/up projection fused with SwiGLU or
 * tanh-GEGLU, then the down projection), and a routing-weighted combine plus an
 * always-on shared expert or parallel dense MLP.  The op split follows the
 * "CANN Qwen3-MoE" page (GMM enablement and routing optimisation: fused top-k
 * softmax, init routing + expert token counts, grouped matmul, finalize routing).
 *
 * Conventions for every entry point
 *  - Tensor pointers are DEVICE pointers to row-major, contiguous storage,
 *    16-byte aligned.  Scalars and structs are host memory.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on it and returns; nothing is copied device->host and no
 *    call synchronises.  Device-side faults surface at the caller's next sync.
 *  - The caller owns every buffer.  The library never allocates or frees
 *    device memory and keeps no per-call state, so calls on different streams
 *    are independent as long as their output and workspace buffers are
 *    disjoint.  The one piece of library state is the optional stage timing
 *    record (moe_timing_enable / moe_timing_read), which belongs to the host
 *    thread that enables it.
 *  - Errors are return values (moe_status_t).  Nothing throws, aborts or
 *    prints.  Validation is synchronous and happens before anything is
 *    enqueued; a failed launch returns MOE_ERR_LAUNCH.
 *  - Weight layout is [out, in]: W13[e] is [2I, D] with rows [0,I) the gate
 *    projection and rows [I,2I) the up projection (the concatenated w13 of the
 *    CANN Qwen3-MoE page, whose swiglu applies SiLU to the first half of the
 *    chunked product); W2[e] is [D, I].  fp8 weights carry fp32 per-output-
 *    channel scales s13[e][2I] and s2[e][D], applied after the reduction
 *    ("Ling-2.6-1T with SGLang-JAX" page, section 5, per-channel scaling).
 *    MXFP4 weights carry E8M0 block scales in place of the per-channel ones:
 *    s13[e] is uint8 [D/128][2I][4] and s2[e] uint8 [I/128][D][4] (for each
 *    group of 128 K elements, each output row's four block scales side by
 *    side).
 *  - Supported dtype combinations: {act F32, weights F32},
 *    {act BF16, weights BF16 or FP8_E4M3FN}, the latter also with dynamic
 *    per-token fp8 activations (act_quant), and {act BF16, routed and shared
 *    weights MXFP4_E2M1, act_quant MXFP8} (W4A8); anything else is
 *    MOE_ERR_UNSUPPORTED (no silent fallback).
 *  - Limits: 1 <= k <= min(E, 32); E <= 1024; D, I, I_shared multiples of 64;
 *    T*k below 2^31 and the launch grids within int32 ((T*k/16 + T/16 + E + 2)
 *    * (max(D, I, I_shared, E)/64 + 1) below 2^31).  Element offsets are
 *    64-bit; the LDS-tiled GEMM
 *    addresses each activation operand (x, h) and each expert's weights with
 *    32-bit byte offsets, so where one of them reaches 4 GiB the layer runs
 *    the register-streamed GEMM instead (with act_quant, which needs the
 *    tiled GEMM: MOE_ERR_SHAPE).  T == 0 is valid and enqueues nothing.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtypes */
#define MOE_F32         0
#define MOE_BF16        1
#define MOE_FP8_E4M3FN  2   /* OCP e4m3fn: bias 7, max 448, no inf, 0x7F/0xFF NaN */
#define MOE_MXFP4_E2M1  3   /* weights only: OCP MXFP4, e2m1 codes two per byte
                               (element 2j in the low nibble) with one E8M0
                               scale 2^(e-127) per 32 consecutive K elements */

/* gated activations of the expert FFN */
#define MOE_ACT_SILU       0   /* SwiGLU: SiLU(gate) * up            */
#define MOE_ACT_GELU_TANH  1   /* GEGLU:  tanh-GELU(gate) * up       */

/* tile policies of the grouped FFN */
#define MOE_TILE_AUTO     0    /* chosen on the host from T*k/E, the weight
                                  format and the sizes (decode batches: 32-row
                                  LDS-tiled blocks; prefill: 128 / 256-row)  */
#define MOE_TILE_STREAM   1    /* register-streamed weights, no LDS         */
#define MOE_TILE_LDS      2    /* LDS-tiled MFMA GEMM, 128 / 256-row tiles   */

/* activation quantisation of the expert GEMMs (moe_problem_t.act_quant) */
#define MOE_ACT_QUANT_NONE     0   /* bf16 activations                       */
#define MOE_ACT_QUANT_FP8_ROW  1   /* dynamic per-token fp8 (see below)      */
#define MOE_ACT_QUANT_MXFP8    2   /* dynamic MXFP8 blocks (see below)       */
#define MOE_ACT_QUANT_FP8_SUB  3   /* dynamic fp8 per 512-column slice (below) */
#define MOE_SUBCHANNEL       512   /* slice width of MOE_ACT_QUANT_FP8_SUB    */

/* where moe_layer combines the expert rows (moe_problem_t.combine) */
#define MOE_COMBINE_AUTO      0    /* the library's choice: separate (measured
                                      faster on every layer, see moe_layer)   */
#define MOE_COMBINE_SEPARATE  1    /* a combine launch after the down projection */
#define MOE_COMBINE_FUSED     2    /* in the down projection where it allows it,
                                      else separate (see moe_layer)           */

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,          /* a required pointer is NULL               */
  MOE_ERR_SHAPE = 2,         /* a size is out of the supported range     */
  MOE_ERR_DTYPE = 3,         /* an unknown dtype / activation code       */
  MOE_ERR_UNSUPPORTED = 4,   /* a valid but unsupported combination      */
  MOE_ERR_WORKSPACE = 5,     /* workspace smaller than required          */
  MOE_ERR_LAUNCH = 6         /* a kernel launch or HIP runtime call failed */
} moe_status_t;

/* Problem description (host struct, plain int32 fields). */
typedef struct moe_problem {
  int32_t T;              /* tokens                                          */
  int32_t D;              /* hidden size                                     */
  int32_t E;              /* routed experts                                  */
  int32_t k;              /* experts per token                               */
  int32_t I;              /* routed expert intermediate size                 */
  int32_t I_shared;       /* shared expert / dense MLP intermediate, 0 = none */
  int32_t act;            /* MOE_ACT_* of the routed experts                 */
  int32_t act_shared;     /* MOE_ACT_* of the shared branch                  */
  int32_t renormalize;    /* 1: top-k weights renormalised to sum 1; 0: the
                             selected experts' softmax probabilities over all E
                             experts ("TP MoE" page, 3.3: softmax gating) */
  int32_t act_dtype;      /* x, router weight, h, o and y: MOE_F32 | MOE_BF16 */
  int32_t w_dtype;        /* routed W13 / W2                                 */
  int32_t shared_w_dtype; /* shared W13s / W2s                               */
  int32_t tile_policy;    /* MOE_TILE_*                                      */
  int32_t act_quant;      /* MOE_ACT_QUANT_*: activations of the expert GEMMs */
  int32_t combine;        /* MOE_COMBINE_*: moe_layer only                   */
} moe_problem_t;

/*
 * act_quant (grouped FFN and fused layer):
 *  MOE_ACT_QUANT_NONE     bf16 activations (weights decoded exactly; W8A16
 *                         with fp8 weights).
 *  MOE_ACT_QUANT_FP8_ROW  dynamic per-token fp8 activations, the activation
 *                         quantisation of the "Ling-2.6-1T with SGLang-JAX"
 *                         page, section 5: each GEMM input row (x for the
 *                         gate/up projection, the stored bf16 h for the down
 *                         projection) is quantised as moe_quantize_rows does,
 *                         multiplied with the fp8 weights on the fp8 matrix
 *                         cores (fp32 sums), and scaled per row and per output
 *                         channel after the reduction.  Requires act BF16,
 *                         fp8 routed (and shared) weights, D, I and I_shared
 *                         multiples of 128 and a tile policy other than
 *                         MOE_TILE_STREAM; routing and combine are unchanged.
 *                         Results differ from the exact layer by the
 *                         quantisation (a few per cent of the output range).
 *  MOE_ACT_QUANT_MXFP8    W4A8 ("CANN Qwen3-MoE" page, high-throughput
 *                         prefill: MXFP4 weights, activations quantised
 *                         dynamically to MXFP8 before the grouped matmul):
 *                         each GEMM input row (x; the stored bf16 h) is
 *                         quantised as moe_quantize_rows_mx does, and the
 *                         e4m3fn blocks and the MXFP4 weight blocks are
 *                         multiplied on the scaled fp8/fp4 matrix cores with
 *                         both block scales applied inside the product.
 *                         Requires act BF16, MXFP4 routed and shared weights,
 *                         D, I and I_shared multiples of 128 and a tile policy
 *                         other than MOE_TILE_STREAM.
 *  MOE_ACT_QUANT_FP8_SUB  as MOE_ACT_QUANT_FP8_ROW with one scale per
 *                         MOE_SUBCHANNEL-column slice of each row instead of
 *                         one per row: the 512 sub-channel activation
 *                         quantisation of the fp8 grouped matmul on the "Qwen
 *                         3.5 MoE on Ironwood" page (MoE track, GMM v2).  Each
 *                         GEMM input row (x; the stored bf16 h) is quantised
 *                         as moe_quantize_subchannel does; the row's sum is
 *                         sum over slices j of s_j times the slice's fp8
 *                         products (fp32 sums; the slice scale's power of two
 *                         is applied by the matrix cores, its mantissa by
 *                         rescaling the partial sums at each slice boundary),
 *                         then scaled per output channel.  Requires what
 *                         MOE_ACT_QUANT_FP8_ROW requires, with D, I and
 *                         I_shared multiples of 512.
 */

/*
 * moe_route -- router logits and top-k softmax gating.
 *   logits = x . Wr^T accumulated in fp32 ("Qwen 3.5 MoE on Ironwood", model
 *   architecture: the router projects the token and takes a softmax; the CANN
 *   Qwen3-MoE page feeds the gate fp32 activations), then per token the k
 *   largest logits in descending order, equal values going to the lower expert
 *   index, weighted w_j = exp(l_j - l_0) / sum_m exp(l_m - l_0): the
 *   renormalised top-k of the softmax, done as one fused op as on the CANN
 *   Qwen3-MoE page (fused top-k softmax).
 *   x        [T, D] act dtype           (unused if logits_given)
 *   w_router [E, D] act dtype           (unused if logits_given)
 *   logits   [T, E] fp32: written, or read when logits_given != 0
 *   topk_idx [T, k] int32 written;  topk_w [T, k] fp32 written
 */
moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* w_router,
                       float* logits, int32_t logits_given, int32_t* topk_idx,
                       float* topk_w, void* stream);

/*
 * moe_permute -- per-expert token counts and the stable expert-major
 * permutation ("init routing" and "compute expert tokens" on the CANN
 * Qwen3-MoE page), and optionally the contiguous permuted copy of the tokens
 * (the gather into one buffer of the SparseCore path on the Ironwood page, MoE
 * track).
 *   topk_idx    [T, k] int32, each row k distinct ids in [0, E)
 *   counts      [E]    rows routed to each expert
 *   offsets     [E+1]  exclusive prefix sum of counts (offsets[E] = T*k)
 *   row_token   [T*k]  token of each sorted row; rows of one expert are in
 *                      ascending token order
 *   row_of_slot [T*k]  sorted row of assignment (t, j) at index t*k + j
 *   x, x_perm          both NULL, or both given: x [T, D] act dtype and
 *                      x_perm [T*k, D] act dtype, 16-byte aligned; then
 *                      x_perm[r] = x[row_token[r]] for r < offsets[E] (rows
 *                      past it are not written).  moe_grouped_ffn can read
 *                      x_perm directly (row_token = NULL); the fused layer
 *                      gathers inside its GEMM instead and never builds it.
 *   ws / ws_bytes      scratch of at least moe_permute_workspace_size bytes
 * Deterministic: no order-dependent atomics.  Ids outside [0, E) are a
 * caller error: they are dropped (row_of_slot = -1) and counts then sum to
 * less than T*k; repeated ids within a row are a caller error too.  Exactly
 * one of x / x_perm NULL is MOE_ERR_NULL; a misaligned one MOE_ERR_SHAPE.
 */
moe_status_t moe_permute_workspace_size(const moe_problem_t* p, size_t* bytes);
moe_status_t moe_permute(const moe_problem_t* p, const int32_t* topk_idx, int32_t* counts,
                         int32_t* offsets, int32_t* row_token, int32_t* row_of_slot, const void* x,
                         void* x_perm, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_grouped_ffn -- grouped gated expert FFN over n_groups experts.
 *   For group g and its rows r in [offsets[g], offsets[g+1]):
 *     [gate | up] = A_r . W13[g]^T  (x s13[g] after the reduction for fp8),
 *     h_r = act(gate) * up,  out_r = h_r . W2[g]^T  (x s2[g] for fp8)
 *   ("CANN Qwen3-MoE", MoE TP compute decomposition: x = down(SiLU(gate(x)) *
 *   up(x)) with gate/up merged into w13; grouped matmul over many experts in
 *   one call; "Gemma-4 model optimisation report" section 2 for GEGLU.)
 *   The problem's D, I, act, act_dtype, w_dtype and tile_policy describe this
 *   call (pass I = I_shared and act = act_shared to run a shared branch as one
 *   group with offsets {0, T} and row_token = NULL).
 *   a         [*, D] act dtype: A_r = a[row_token[r]] if row_token, else a[r]
 *   row_token [rows] int32 or NULL
 *   offsets   [n_groups+1] int32 device array, offsets[n_groups] <= rows_upper_bound
 *   w13 [n_groups, 2I, D], w2 [n_groups, D, I] (w_dtype; MXFP4: D/2 and I/2
 *   bytes per row); s13 [n_groups, 2I], s2 [n_groups, D] fp32 for fp8, the
 *   E8M0 block scales for MXFP4 (layout above), ignored otherwise
 *   h   [rows_upper_bound, I] act dtype (written; intermediate)
 *   out [rows_upper_bound, D] act dtype (written)
 *   rows_upper_bound  host-known bound on offsets[n_groups]; it sizes the grid;
 *                     rows_upper_bound * max(D, I) below 2^31, else MOE_ERR_SHAPE
 *   ws / ws_bytes     scratch of at least moe_grouped_ffn_workspace_size bytes
 *   With act_quant the quantised copies of the A rows and of h (and their
 *   scales) live in the workspace; h is still written in bf16 (it is the
 *   stored value that gets quantised).
 */
moe_status_t moe_grouped_ffn_workspace_size(const moe_problem_t* p, int32_t n_groups,
                                            int32_t rows_upper_bound, size_t* bytes);
moe_status_t moe_grouped_ffn(const moe_problem_t* p, int32_t n_groups, int32_t rows_upper_bound,
                             const void* a, const int32_t* row_token, const int32_t* offsets,
                             const void* w13, const void* s13, const void* w2, const void* s2,
                             void* h, void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine -- unpermute and routing-weighted sum ("finalize routing" on the
 * CANN Qwen3-MoE page; the unpermute + local reduce of the Ironwood page's MoE
 * track), plus the shared branch:
 *   y[t] = sum_{j<k} topk_w[t,j] * o_perm[row_of_slot[t*k+j]] + shared_out[t]
 *   accumulated in fp32 in slot order, rounded once to the act dtype.
 *   o_perm [T*k, D], shared_out [T, D] or NULL, y [T, D]: act dtype.
 *   Assignments whose row_of_slot is negative or not below T*k contribute
 *   nothing.
 */
moe_status_t moe_combine(const moe_problem_t* p, const void* o_perm, const int32_t* row_of_slot,
                         const float* topk_w, const void* shared_out, void* y, void* stream);

/* Arguments of the fused layer.  Optional outputs (NULL = not wanted) are
 * written when given; logits_in (nullable) replaces the router product. */
typedef struct moe_layer_args {
  const void* x;            /* [T, D] act dtype                          */
  const void* w_router;     /* [E, D] act dtype (unused with logits_in)  */
  const float* logits_in;   /* [T, E] fp32 or NULL                        */
  const void* w13;          /* [E, 2I, D]                                 */
  const void* s13;          /* [E, 2I] fp32 (fp8); E8M0 blocks (MXFP4)    */
  const void* w2;           /* [E, D, I]                                  */
  const void* s2;           /* [E, D]  fp32 (fp8); E8M0 blocks (MXFP4)    */
  const void* w13_shared;   /* [2I_shared, D]  (NULL iff I_shared == 0)   */
  const void* s13_shared;   /* [2I_shared]     (fp8; MXFP4 blocks)        */
  const void* w2_shared;    /* [D, I_shared]                              */
  const void* s2_shared;    /* [D]             (fp8; MXFP4 blocks)        */
  void* y;                  /* [T, D] act dtype, written                  */
  float* logits_out;        /* [T, E] optional                            */
  int32_t* topk_idx_out;    /* [T, k] optional                            */
  float* topk_w_out;        /* [T, k] optional                            */
  int32_t* counts_out;      /* [E]    optional                            */
  int32_t* offsets_out;     /* [E+1]  optional                            */
  int32_t* row_token_out;   /* [T*k]  optional                            */
  int32_t* row_of_slot_out; /* [T*k]  optional                            */
} moe_layer_args_t;

/*
 * moe_layer -- the whole layer, every step enqueued on one stream with no
 * host synchronisation: route -> permute -> grouped FFN (routed experts and the
 * shared branch in the same launches) -> combine.  The workspace holds every
 * intermediate (logits, routing metadata, h, o, the combine's arrival
 * counters, and with act_quant the fp8 copies of x and h with their row
 * scales); its size depends only on the problem.
 *   Combine: with MOE_COMBINE_FUSED, and where the down projection runs on
 *   the LDS-tiled kernel with bf16 rows in one launch (bf16 activations,
 *   routed and shared weights of one dtype), the combine runs inside the
 *   down projection: each token is combined by the block that stores its
 *   last expert row of a column block (owner computes, as the single-point
 *   accumulation per token of the "Gemma-4 model optimisation report",
 *   section 5.3), with the arithmetic of moe_combine (fp32 in slot order,
 *   the shared row last, one rounding), so y is bit-identical to the
 *   separate combine's.  Elsewhere, and with MOE_COMBINE_SEPARATE or
 *   _AUTO, a moe_combine launch follows the down projection: the expert
 *   rows have to cross between the GPU's XCDs (each with its own L2) either
 *   way, and the fused form's device-scope stores and end-of-block counting
 *   cost more than the separate launch (Ling decode layer 2.53 vs 2.41 ms,
 *   Ling prefill 16.8 vs 14.4 ms, measured).
 */
moe_status_t moe_layer_workspace_size(const moe_problem_t* p, size_t* bytes);
moe_status_t moe_layer(const moe_problem_t* p, const moe_layer_args_t* args, void* ws,
                       size_t ws_bytes, void* stream);

/*
 * moe_layer_noalloc -- moe_layer for callers that cannot allocate device
 * memory (work under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same launches, with the workspace in a device array
 * owned by the library (moe_layer_noalloc_max_bytes() bytes, 128 MiB, held
 * on every GPU the library runs on until the process ends) instead of a
 * caller buffer.  The caller still passes the inputs and outputs (args).
 * Nothing is allocated: no hipMalloc, hipFree or allocating library call, and
 * no timing events (stage timing is not recorded for these calls).
 *   Problems whose moe_layer_workspace_size exceeds the array return
 *   MOE_ERR_WORKSPACE before anything is enqueued (the decode-sized layers
 *   fit: 9 MiB for 64 tokens of the Qwen3.5 layer, 106 MiB for 512 tokens of
 *   the Ling layer; prefill-sized ones do not).
 *   The array belongs to the device of `stream`, and every call on that
 *   device shares it: calls that overlap on one device (concurrent streams,
 *   or host threads) race on it and must be serialised by the caller.  It
 *   keeps the last call's contents; nothing in it needs to start at zero.
 *   Other errors are those of moe_layer; MOE_ERR_LAUNCH also covers a failure
 *   to look up the array's device address.
 */
size_t moe_layer_noalloc_max_bytes(void);
moe_status_t moe_layer_noalloc(const moe_problem_t* p, const moe_layer_args_t* args, void* stream);

/*
 * moe_quantize_rows -- dynamic per-row fp8 quantisation ("Ling-2.6-1T with
 * SGLang-JAX" page, section 5, activation quantisation): for each row r,
 *   scale[r] = max_c |a[r][c]| / 448 in fp32 (448 = largest finite e4m3fn
 *              magnitude; 1 for a row of zeros), and
 *   q[r][c]  = the e4m3fn code nearest to a[r][c] / scale[r] (fp32 division),
 *              ties to the even code, magnitudes above 448 saturating to 448,
 *              the sign bit kept (so -0 and tiny negatives give 0x80).
 *   a     [rows, lda] bf16 (the first cols columns are read); lda % 8 == 0
 *   q     [rows, cols] uint8 (written);  scale [rows] fp32 (written)
 *   cols % 8 == 0 and 0 < cols <= 16384, else MOE_ERR_SHAPE; a 16-byte and q
 *   8-byte aligned.  Non-finite inputs are outside the contract.
 */
moe_status_t moe_quantize_rows(const void* a, int32_t rows, int32_t cols, int64_t lda, uint8_t* q,
                               float* scale, void* stream);

/*
 * moe_quantize_subchannel -- dynamic fp8 quantisation per 512-column slice
 * (the sub-channel activation quantisation of the "Qwen 3.5 MoE on Ironwood"
 * page, MoE track, GMM v2): moe_quantize_rows' rule applied to each slice of
 * MOE_SUBCHANNEL consecutive columns of a row, with its own scale.
 *   a     [rows, lda] bf16 (the first cols columns are read); lda % 8 == 0
 *   q     [rows, cols] uint8 (written)
 *   scale [cols / 512, rows] fp32 (written, slice-major: the scale of row r's
 *         slice u at scale[u * rows + r])
 *   cols % 512 == 0 and 0 < cols <= 16384, else MOE_ERR_SHAPE; a 16-byte and
 *   q 8-byte aligned.  Non-finite inputs are outside the contract.
 */
moe_status_t moe_quantize_subchannel(const void* a, int32_t rows, int32_t cols, int64_t lda, uint8_t* q,
                                     float* scale, void* stream);

/*
 * moe_quantize_rows_mx -- dynamic MXFP8 quantisation, the activation side of
 * the W4A8 decomposition ("CANN Qwen3-MoE" page, high-throughput prefill),
 * with the block format of the OCP microscaling specification: each block of
 * 32 consecutive elements of a row gets one E8M0 scale code
 *   e = clamp(floor(log2(max |a|)) - 8, -127, 127) + 127   (8 = the largest
 *       e4m3fn exponent; a block of zeros gets e = 0),
 * and each element the e4m3fn code nearest to a / 2^(e-127) (exact power-of-
 * two scaling), ties to the even code, magnitudes above 448 saturating.
 *   a     [rows, lda] bf16 (the first cols columns are read); lda % 8 == 0
 *   q     [rows, cols] uint8 (written)
 *   scale uint8 [cols/128][rows][4] (written): the scale of block b of row r
 *         at (b / 4) * rows * 4 + r * 4 + b % 4, the layout the W4A8 GEMM reads
 *   cols % 128 == 0 and 0 < cols <= 16384, else MOE_ERR_SHAPE; a 16-byte and q
 *   8-byte aligned.  Non-finite inputs are outside the contract.
 */
moe_status_t moe_quantize_rows_mx(const void* a, int32_t rows, int32_t cols, int64_t lda, uint8_t* q,
                                  uint8_t* scale, void* stream);

/*
 * The kernel shape each product of moe_layer takes for a problem: the planning
 * moe_layer itself runs, on the host only (no device call; callable without a
 * GPU).  For tests and tools that need to know which path a problem covers.
 *   router / gate_up / down   a moe_plan_shape_t (the router is planned even
 *                             when the caller passes logits in);
 *   router_slices             K slices of the router product, whose fp32
 *                             partial sums the top-k step adds in slice order;
 *   one_launch_permute        1 when the permutation and the M-tile table run
 *                             as one launch, else 0.
 * Returns the status moe_layer_workspace_size returns for p, or MOE_ERR_NULL
 * for a null out.
 */
typedef enum {
  MOE_PLAN_STREAM_16 = 0,       /* register-streamed GEMM, 16-row tiles */
  MOE_PLAN_STREAM_32 = 1,       /* ... 32-row tiles */
  MOE_PLAN_STREAM_64 = 2,       /* ... 64-row tiles */
  MOE_PLAN_TILED_256x256 = 3,   /* LDS-tiled GEMM, rows x weight rows per block */
  MOE_PLAN_TILED_128x512 = 4,
  MOE_PLAN_TILED_128x256 = 5,
  MOE_PLAN_TILED_32x128 = 6,
  MOE_PLAN_TILED_64x256 = 7,
  MOE_PLAN_TILED_32x64 = 8
} moe_plan_shape_t;
typedef struct moe_plan {
  int32_t router, router_slices, gate_up, down, one_launch_permute;
} moe_plan_t;
moe_status_t moe_layer_plan(const moe_problem_t* p, moe_plan_t* out);

/* Human-readable name of a status code (static string; "unknown status" for
 * any other value). */
const char* moe_status_string(moe_status_t status);

/*
 * Per-stage kernel timing with HIP events, for measurement.  While enabled,
 * moe_layer (and the stage entry points) record an event pair around each
 * selected stage on their stream.  moe_timing_enable(on): on = 0 disables,
 * on > 0 selects every stage, and on < 0 selects the stages whose bits are set
 * in on & 0x7fffffff (bit s = stage s; e.g. (int32_t)(0x80000000u | (1u << 4))
 * times only the gate/up projection, which keeps the events' own cost out of
 * the other stages).  moe_timing_read waits for the recorded events, adds each stage's
 * elapsed time (ms) and launch count into ms[stage] / launches[stage] for
 * stage < n_stages, and clears the record.  Stage names: moe_stage_name.
 * The record (enable flag, stage mask, pending events) is per host thread:
 * enabling timing on one thread does not time calls made on another, and
 * moe_timing_read returns the calling thread's stages only.
 */
moe_status_t moe_timing_enable(int32_t on);
moe_status_t moe_timing_read(double* ms, int32_t* launches, int32_t n_stages);
int32_t moe_stage_count(void);
const char* moe_stage_name(int32_t stage);

/*
 * Measurement probes (not part of the layer): the ceilings the benchmark
 * reports next to the published peaks, measured on the part it runs on.
 *  moe_probe_hbm_read   streams `bytes` (a multiple of 16, buf 16-byte
 *                       aligned) from buf with eight 16-byte non-temporal
 *                       loads in flight per thread; sink [1024] uint32 is
 *                       written only if a data-dependent fold hits a magic
 *                       value (it exists so the loads cannot be dropped).
 *  moe_probe_mfma       independent register-only MFMAs, iters rounds per
 *                       wavefront, on operands read from 64 KiB at `operands`
 *                       (finite values of the probe's type: bf16 for MOE_BF16,
 *                       the bf16 GEMMs' 16x16x32 instruction; e4m3fn codes for
 *                       MOE_FP8_E4M3FN, the fp8 x fp8 GEMM's 32x32x64 one);
 *                       *flop (host) receives the launch's FLOP count; sink
 *                       holds moe_probe_mfma_sink_floats() floats.
 * Time them with events on `stream`.
 */
moe_status_t moe_probe_hbm_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);
int32_t moe_probe_mfma_sink_floats(void);
moe_status_t moe_probe_mfma(int32_t dtype, const void* operands, int32_t iters, float* sink,
                            double* flop, void* stream);

/*
 * Diagnostic: decode n (a multiple of 8) fp8 e4m3fn codes to bf16 bit
 * patterns with the exact device routine the grouped FFN uses for fp8
 * weights, so the hardware conversion can be checked code by code against the
 * format definition.  codes [n] uint8, out [n] uint16 (device pointers).
 */
moe_status_t moe_debug_fp8_to_bf16(const uint8_t* codes, uint16_t* out, int32_t n, void* stream);

/*
 * Diagnostic: encode n (even) fp32 values, each clamped to +-448 first, to
 * fp8 e4m3fn codes (nearest representable value, ties to the even code) with
 * the exact device routine the activation quantisers use, so the hardware
 * conversion can be checked against the format definition.  v [n] float,
 * out [n] uint8 (device pointers).  Non-finite inputs are outside the
 * contract.
 */
moe_status_t moe_debug_f32_to_fp8(const float* v, uint8_t* out, int32_t n, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
