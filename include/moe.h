/*
 * moe.h - C ABI of the one-GPU share of an expert-parallel MoE layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (Perplexity, "Lower latency and higher throughput with multi-node
 * DeepSeek deployment", section Expert parallelism): every token is sent to
 * its top-K routed experts, the expert outputs are summed with the router
 * weights, and a shared expert present on every GPU adds its output. Under
 * expert parallelism a GPU holds E/EP routed experts; here the other ranks are
 * logical source partitions of one global batch held on this GPU.
 *
 * Pipeline, one call per step, all enqueued on the caller's stream:
 *   moe_route_topk       top-K experts and weights per token
 *   moe_dispatch_layout  per-expert counts, prefix sum, a slot per (token, k)
 *   moe_dispatch         copy token rows into the expert-grouped buffer
 *   moe_grouped_gemm     SwiGLU FFN per local expert (and the shared expert)
 *   moe_combine          weighted sum back in token order
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers unless stated; descriptors and return values
 *    are host memory. The caller allocates and owns every buffer; the library
 *    allocates and frees nothing. Scratch comes in through `ws` with a size
 *    query. Buffers must not alias unless stated.
 *  - Row-major storage; activation rows must be 16-byte aligned
 *    (hidden * element size % 16 == 0 and 16-byte aligned base pointers).
 *  - Every call enqueues on `stream` (NULL = the default stream) and returns
 *    without synchronising. Argument errors are found on the host and
 *    returned before anything is enqueued (MOE_ERR_INVALID_ARG,
 *    MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE); a failed launch returns
 *    MOE_ERR_HIP. Data-dependent conditions (a count above capacity) are
 *    reported through a device status word; kernels never write out of bounds
 *    even when device-side inputs (indices, offsets, counts) are invalid.
 *  - Results are deterministic: no floating-point atomics anywhere, and the
 *    integer layout is bit-reproducible.
 *  - No global mutable state apart from a per-device cache of the compute-unit
 *    count and, for moe_dispatch_layout_noalloc only, its per-GPU scratch
 *    array and the cached address of it; calls from several host threads are
 *    safe (except overlapping moe_dispatch_layout_noalloc calls on one GPU).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* a null pointer with a nonzero size, a size out of range, misalignment */
  MOE_ERR_UNSUPPORTED = 2, /* a valid request this build does not implement (dtype pair, shape limit) */
  MOE_ERR_WORKSPACE = 3,   /* ws is NULL or smaller than the size query returned */
  MOE_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} moe_status_t;

typedef enum {
  MOE_F32 = 0,
  MOE_BF16 = 1,
  MOE_FP8_E4M3 = 2 /* OCP e4m3fn: bias 7, no infinities, max 448 (the gfx950 FP8 format) */
} moe_dtype_t;

typedef enum {
  /* Count-first ragged buffer: rows packed by local expert, then by global
   * token index (lehuy.net, "Decoding high-performance EP kernels", section
   * Throughput: ask first, send later > Dispatch; Perplexity, "Enabling
   * trillion-parameter models on AWS EFA", section Send and receive buffers). */
  MOE_LAYOUT_COMPACT = 0,
  /* Fixed rectangle: a private region of `capacity` rows per (local expert,
   * source rank), expert-major, static address (lehuy.net page, section
   * Latency: send without asking). */
  MOE_LAYOUT_PADDED = 1
} moe_layout_t;

/* Storage of an activation matrix [R, K] (bf16, K % 32 == 0).
 * ROWS: row-major. BLOCKED16: blocks of 16 rows x 32 columns (1 KiB) stored
 * contiguously, the blocks of one 16-row group in column order: element
 * (r, c) sits at ((r / 16) * (K / 32) + c / 32) * 512 + (r % 16) * 32 + c % 32.
 * A blocked matrix holds ceil(R / 16) * 16 rows. The grouped GEMM loads
 * 16 rows x 32 columns per wave instruction; blocked, that is one contiguous
 * KiB instead of 16 separate 64-byte pieces. */
typedef enum {
  MOE_ACT_ROWS = 0,
  MOE_ACT_BLOCKED16 = 1
} moe_act_layout_t;

/* Bit of the device status word written by moe_dispatch_layout. */
#define MOE_STATUS_OVERFLOW 1

/* Library version and a readable name for a status code (static strings). */
int moe_abi_version(void);
const char* moe_status_string(moe_status_t s);

/* ------------------------------------------------------------------ route
 * Top-K routing (Perplexity DeepSeek deployment page, section MoE Router:
 * the router yields top-K expert indices and scores per token; the softmax
 * rule is the plain, group-free case the page calls Mixtral's).
 *
 * logits    [n_tokens, n_experts] float32.
 * topk_idx  [n_tokens, top_k] int32 out: experts by descending logit, equal
 *           logits broken by the lower expert index (+0 and -0 compare equal).
 * topk_w    [n_tokens, top_k] float32 out: softmax(logits)[idx], divided by
 *           its sum over the K picked when renormalize != 0.
 * Limits: 1 <= n_experts <= 1024, 1 <= top_k <= min(16, n_experts),
 *         n_tokens >= 0 (0 enqueues nothing). NaN logits give unspecified
 *         but in-range indices.
 */
moe_status_t moe_route_topk(const float* logits, int n_tokens, int n_experts, int top_k, int renormalize,
                            int32_t* topk_idx, float* topk_w, hipStream_t stream);

/* ------------------------------------------------------------------ layout */
typedef struct {
  int n_tokens;     /* N = sum of B_s */
  int top_k;        /* K */
  int n_experts;    /* E (global) */
  int n_src;        /* S logical source ranks, 1..4096 */
  int expert_lo;    /* first local expert */
  int n_local;      /* L local experts [expert_lo, expert_lo + L), 1..1024, L*S <= 65536 */
  moe_layout_t layout;
  int capacity;     /* COMPACT: rows available in the expert buffer (worst case N*min(K,L));
                       PADDED: rows per (expert, source) region (max B_s never overflows) */
} moe_layout_desc_t;

/* Rows R of the expert-grouped buffer (xe, ye, h): COMPACT capacity,
 * PADDED n_local * n_src * capacity. Returns -1 for an invalid descriptor. */
int64_t moe_layout_rows(const moe_layout_desc_t* d);

/* Bytes of scratch moe_dispatch_layout needs; 0 for an invalid descriptor. */
size_t moe_dispatch_layout_workspace(const moe_layout_desc_t* d);

/* Per-expert aggregation of the routing and a slot for every (token, k)
 * (Perplexity DeepSeek page, section MoE Router: all-to-all dispatch needs the
 * routing per expert; AWS EFA page, section Dispatch and combine: per-expert
 * counts, then their prefix sum gives the offsets; lehuy.net page: the
 * prefix sum of the counts is the layout, or a static stride times a fixed
 * maximum in the fixed-rectangle shape).
 *
 * topk_idx    [N, K] int32 (any values; those outside the local range are
 *             not local).
 * src_offsets [S + 1] int32: source s owns tokens [src_offsets[s],
 *             src_offsets[s+1]); must start at 0, be nondecreasing and end at
 *             N (other values are clamped into that shape).
 * counts      [L, S] int32 out: entries of source s routed to local expert le
 *             (before any capacity drop), at counts[le * S + s].
 * expert_off  [L + 1] int32 out: first row of each local expert. COMPACT:
 *             exclusive prefix sum of the per-expert totals, clipped to
 *             capacity (expert_off[L] = rows in use). PADDED: le * S * capacity.
 * row_of      [N * K] int32 out: row of entry (t, k) at t*K + k, or -1 (not
 *             local, or dropped). COMPACT rows inside one expert follow the
 *             token order; PADDED entry j of (le, s) sits at
 *             (le * S + s) * capacity + j.
 * row_token   [R] int32 out: token held by each row, -1 for an unused row.
 * status      [1] int32 out: MOE_STATUS_OVERFLOW if a row had to be dropped
 *             (COMPACT: total above capacity; PADDED: a count above capacity).
 * ws          scratch of moe_dispatch_layout_workspace(d) bytes.
 */
moe_status_t moe_dispatch_layout(const moe_layout_desc_t* d, const int32_t* topk_idx, const int32_t* src_offsets,
                                 int32_t* counts, int32_t* expert_off, int32_t* row_of, int32_t* row_token,
                                 int32_t* status, void* ws, size_t ws_bytes, hipStream_t stream);

/* moe_dispatch_layout without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments and results as
 * moe_dispatch_layout; the scratch is a fixed 4 MiB array in the library's
 * device data, one copy per GPU, held until the process ends. The call itself
 * allocates and frees nothing. Requests whose workspace
 * (moe_dispatch_layout_workspace) exceeds 4 MiB return MOE_ERR_UNSUPPORTED
 * before anything is enqueued. Every call on one GPU shares that GPU's array:
 * calls that overlap in time on one GPU (several streams, several host
 * threads) race and give undefined results; calls ordered on one stream are
 * safe (each call writes every scratch word it reads). Returns MOE_ERR_HIP if
 * the array's device address cannot be found. */
moe_status_t moe_dispatch_layout_noalloc(const moe_layout_desc_t* d, const int32_t* topk_idx,
                                         const int32_t* src_offsets, int32_t* counts, int32_t* expert_off,
                                         int32_t* row_of, int32_t* row_token, int32_t* status, hipStream_t stream);

/* ------------------------------------------------------------------ dispatch
 * Copy each token row into every slot the layout gave it: xe[row_of[t*K+k]] =
 * x[t] for row_of >= 0 (lehuy.net page, section Throughput > Dispatch: gather
 * the tokens bound for local experts into one buffer the grouped GEMM reads
 * at once). Bit-exact copy; unused rows of xe are not written. Each token row
 * is read once. Entries outside [0, n_rows) are skipped.
 *
 * x [n_tokens, hidden] of dtype dt (MOE_F32 or MOE_BF16); xe [n_rows, hidden].
 */
moe_status_t moe_dispatch(const void* x, moe_dtype_t dt, int n_tokens, int hidden, int top_k,
                          const int32_t* row_of, int64_t n_rows, void* xe, hipStream_t stream);

/* ------------------------------------------------------------------ fp8 payload
 * On-the-fly 1 x 128 quantization of token rows (Perplexity DeepSeek page,
 * section Quantization: activations take one scale per 128-element vector;
 * the dispatch payload is fp8 with its scales, lehuy.net page, section
 * Latency: send without asking, AWS EFA page, section Evaluation). For each
 * row and each block of 128 columns:
 *   s = fp32(max |x|) / 448, and s = 1 where that is 0;
 *   xq = RNE(clamp(fp32(x) / s, -448, 448)) as OCP e4m3fn codes (0x00 for a
 *   zero result), with correctly rounded fp32 division.
 *
 * x  [n_rows, hidden] of dtype dt (MOE_BF16 or MOE_F32), 16-byte aligned.
 * xq [n_rows, hidden] uint8 out (8-byte aligned), xs [n_rows, hidden / 128]
 * float32 out. hidden % 128 == 0 (else MOE_ERR_UNSUPPORTED). NaN inputs give
 * unspecified finite codes.
 */
moe_status_t moe_quantize_1x128(const void* x, moe_dtype_t dt, int64_t n_rows, int hidden, uint8_t* xq, float* xs,
                                hipStream_t stream);

/* moe_dispatch for the fp8 payload: codes and scales of each token row go to
 * every slot the layout gave it (xeq[row_of[t*K+k]] = xq[t], xes[...] =
 * xs[t]); bit-exact; unused rows are not written.
 *
 * xq [n_tokens, hidden] uint8, xs [n_tokens, hidden / 128] float32 (as
 * moe_quantize_1x128 wrote them); xeq [n_rows, hidden], xes [n_rows, hidden /
 * 128]. hidden % 128 == 0; xq and xeq 16-byte aligned.
 */
moe_status_t moe_dispatch_fp8(const uint8_t* xq, const float* xs, int n_tokens, int hidden, int top_k,
                              const int32_t* row_of, int64_t n_rows, uint8_t* xeq, float* xes, hipStream_t stream);

/* The same copy into an expert-grouped buffer in the MOE_ACT_BLOCKED16 layout
 * (same arguments as moe_dispatch): each token row is read once and written to
 * each of its slots' blocks; unused rows are not written.
 *
 * x [n_tokens, hidden] bf16 row-major, hidden % 32 == 0; xe holds
 * ceil(n_rows / 16) * 16 rows of hidden bf16.
 */
moe_status_t moe_dispatch_blocked(const void* x, moe_dtype_t dt, int n_tokens, int hidden, int top_k,
                                  const int32_t* row_of, int64_t n_rows, void* xe, hipStream_t stream);

/* ------------------------------------------------------------------ grouped GEMM */
typedef enum {
  MOE_W_ROWMAJOR = 0, /* w13 [G, 2I, H] and w2 [G, H, I] row-major */
  MOE_W_PACKED = 1    /* the same bytes permuted by moe_pack_weights (bf16 and fp8 only) */
} moe_weight_format_t;

/* Which kernel takes which expert group. Both compute the same products in
 * fp32 (the sum order differs, so results may differ in the last bits).
 * AUTO: if the groups of at least 128 rows make at least 16 tiles of the
 * 256 x 256 wide-tile kernel (bf16 weights, hidden % 256 == 0), every group
 * of the launch takes that kernel, else every group takes the stream-K
 * kernel (decided on the device from the counts). WIDE: every group takes the
 * wide-tile kernel where its shape and dtype allow (then the stream-K kernel
 * is not launched). STREAM_K: never (then the wide kernel is not launched).
 * fp8 weights take the W8A16 or W8A8 kernel whatever the policy; for W8A8,
 * STREAM_K (decode batches) keeps each workgroup's whole tiles contiguous,
 * while AUTO and WIDE let workgroups holding 6 or more whole tiles take every
 * G-th tile instead (prefill batches: neighbouring workgroups then share each
 * weight slab in L2). */
typedef enum {
  MOE_GEMM_AUTO = 0,
  MOE_GEMM_WIDE = 1,
  MOE_GEMM_STREAM_K = 2
} moe_gemm_policy_t;

typedef enum {
  MOE_GG_FULL = 0, /* both products */
  MOE_GG_UP = 1,   /* h = silu(a W_gate^T) * (a W_up^T) into the workspace only */
  MOE_GG_DOWN = 2  /* y = h W2^T from the workspace only (after MOE_GG_UP on the same ws) */
} moe_gg_stage_t;

/* The shared expert (Perplexity DeepSeek page, section Expert parallelism:
 * every GPU keeps a copy of it and runs it on its own tokens). When given,
 * moe_grouped_gemm runs it as one more group inside the same launches as the
 * routed experts, so the small problem does not run alone on a few compute
 * units. Same dtypes and sizes as the routed experts. */
typedef struct {
  const void* a;     /* [rows, H] input rows (act_dt), e.g. this GPU's own tokens */
  int rows;          /* B (0 = no shared expert) */
  const void* w13;   /* [1, 2I, H] */
  const void* w2;    /* [1, H, I] */
  const float* s13;  /* fp8 only: [1, 2I/128, H/128] */
  const float* s2;   /* fp8 only: [1, H/128, I/128] */
  void* y;           /* [rows, H] out (act_dt; bf16 for W8A8) */
  const float* a_scales; /* W8A8 only: [rows, H/128] scales of the codes in a; else NULL */
} moe_shared_expert_t;

/* Weighted scatter from the down projection (lehuy.net page, section
 * Combine; Perplexity DeepSeek page, section Quantization: routing-aware
 * kernels that fuse the grouped GEMM with the data movement around it). A
 * token with exactly one kept entry (one k with row_of[t*K+k] in
 * [0, n_rows)) and no shared-expert row (t outside [self_lo, self_hi)) has
 * that one row as its whole combine; with a scatter, the down projection's
 * epilogue writes
 *   out[t] = round(topk_w[t*K+k] * y[row])   (y first rounded to bf16, the
 *            product formed in fp32 as fmaf(w, y, 0), one rounding)
 * - bit for bit what moe_combine writes for that token - instead of y[row],
 * which is then not written. moe_combine_multi combines the other tokens.
 * bf16 outputs only (bf16 activations or W8A8); device pointers. */
typedef struct {
  const int32_t* row_token; /* [rows] token of each routed row (moe_dispatch_layout) */
  const int32_t* row_of;    /* [n_tokens, top_k] */
  const float* topk_w;      /* [n_tokens, top_k] */
  int n_tokens;
  int top_k;                /* 1..16 */
  int64_t n_rows;           /* the combine's n_rows */
  int self_lo, self_hi;     /* shared-expert token range (equal: none) */
  void* out;                /* [n_tokens, hidden] bf16, 16-byte aligned */
} moe_scatter_t;

typedef struct {
  int n_groups;        /* G routed experts in this call (may be 0 with a shared expert) */
  int hidden;          /* H, multiple of 128 */
  int inter;           /* I, multiple of 128 */
  moe_dtype_t act_dt;  /* a, y, workspace h: MOE_F32 or MOE_BF16; MOE_FP8_E4M3 = W8A8 (see below) */
  moe_dtype_t w_dt;    /* weights: MOE_F32 with f32 activations; MOE_BF16 or MOE_FP8_E4M3 with bf16;
                          MOE_FP8_E4M3 with fp8 activations */
  moe_layout_t layout; /* how rows of a/y are grouped (as moe_dispatch_layout wrote them) */
  int n_src;           /* PADDED: S */
  int capacity;        /* PADDED: rows per (group, source) region */
  int64_t rows;        /* R rows of a, y and h (row indices are shared by all three) */
  moe_gg_stage_t stage;
  const moe_shared_expert_t* shared; /* host pointer, or NULL for none */
  moe_weight_format_t w_format;      /* layout of w13/w2 (and of the shared expert's) */
  moe_gemm_policy_t policy;          /* kernel choice per group; MOE_GEMM_AUTO unless tuning or testing */
  moe_act_layout_t a_layout;         /* storage of the routed rows a (bf16 only for BLOCKED16) */
  /* Gather (NULL = off): routed row r of the up projection's input is row
   * a_rows[r] of a, an [a_nrows, H] row-major bf16 matrix (e.g. the tokens x,
   * with a_rows = row_token from moe_dispatch_layout), so no dispatched copy is
   * needed. Indices are clamped into [0, a_nrows). Needs bf16 activations,
   * MOE_ACT_ROWS and a_nrows * H * 2 <= 2^32. The shared expert, h and y keep
   * their own rows. */
  const int32_t* a_rows;             /* device [rows], or NULL */
  int64_t a_nrows;
  /* W8A8 (act_dt = w_dt = MOE_FP8_E4M3): a holds e4m3fn codes [R, H] (or
   * [a_nrows, H] when gathering) and a_scales one float32 scale per row and
   * 128 columns ([R, H/128], or [a_nrows, H/128]), as moe_quantize_1x128 and
   * moe_dispatch_fp8 write them; NULL otherwise. */
  const float* a_scales;
  /* Weighted scatter of single-row tokens from the down projection (host
   * pointer, or NULL for none); used with MOE_GG_FULL and MOE_GG_DOWN. */
  const moe_scatter_t* scatter;
} moe_ggemm_desc_t;

/* Bytes of scratch moe_grouped_gemm needs (the intermediates h [R, I] and, with
 * a shared expert, [B, I], in the activation dtype (W8A8: codes plus one
 * float32 scale per 128 columns), 256-byte aligned); 0 for an invalid
 * descriptor. */
size_t moe_grouped_gemm_workspace(const moe_ggemm_desc_t* d);

/* Per-expert SwiGLU FFN over the rows each expert holds (Perplexity DeepSeek
 * page, section GroupGEMM: g groups, group i a [m_i, k] x [k, n] product;
 * section Quantization: SiLU activation, fp8 weights with one scale per
 * 128 x 128 tile; routing-aware kernels read per-expert counts on the device
 * instead of sizing work from the buffer bound):
 *   h[r] = silu(W13[g][0:I] a[r]) * (W13[g][I:2I] a[r]),   y[r] = W2[g] h[r]
 * for every occupied row r of group g, with fp32 accumulation; h and y are
 * rounded to the activation dtype. Unoccupied rows are not written. Empty
 * groups cost nothing.
 *
 * a          [R, H] activations (act_dt), stored as desc->a_layout says (the
 *            shared expert's rows are always row-major). The intermediate h
 *            lives in the workspace (bf16: blocked layout).
 * counts     [G, S] int32 (PADDED: group g's rows are, for each s,
 *            (g*S+s)*capacity + [0, min(counts[g*S+s], capacity)) ); may be NULL
 *            for COMPACT.
 * group_off  [G + 1] int32 (COMPACT: group g owns rows [group_off[g],
 *            group_off[g+1])); may be NULL for PADDED.
 * w13        [G, 2I, H]: gate rows 0..I-1, then up rows I..2I-1 (w_dt; fp8 as raw bytes).
 * w2         [G, H, I].
 * s13, s2    fp8 only: float32 scales [G, 2I/128, H/128] and [G, H/128, I/128]; else NULL.
 * y          [R, H] out (act_dt); unused with MOE_GG_UP.
 * The shared expert is either desc->shared (same launches) or a call of its own
 * with n_groups = 1, COMPACT, group_off = {0, B} and a pointing at its rows.
 * MOE_GG_UP then MOE_GG_DOWN with the same workspace equals MOE_GG_FULL.
 *
 * W8A8 (act_dt = w_dt = MOE_FP8_E4M3; Perplexity DeepSeek page, section
 * Quantization): activations and weights both fp8 with block scales, so for
 * each output element and 128-deep block kb of the reduction
 *   out += sa[row, kb] * sw[n / 128, kb] * sum_{k in kb} a_code[row, k] w_code[n, k],
 * accumulated in fp32; h = silu(g) * u is quantized 1 x 128 in the up
 * projection's epilogue (the moe_quantize_1x128 rule on the fp32 h) and the
 * down projection reads those codes; y (and the shared expert's y) is bf16.
 * Needs MOE_ACT_ROWS, a_scales (and shared->a_scales) and 16-byte aligned
 * code rows; 4-byte aligned scales.
 */
moe_status_t moe_grouped_gemm(const moe_ggemm_desc_t* d, const void* a, const int32_t* counts,
                              const int32_t* group_off, const void* w13, const void* w2, const float* s13,
                              const float* s2, void* y, void* ws, size_t ws_bytes, hipStream_t stream);

/* One-time permutation of expert weights into the order the grouped-GEMM
 * kernel streams them (weights are static, quantized and stored once;
 * Perplexity DeepSeek page, section Quantization). For expert g, block nt of
 * 128 weight rows (W13: the gate and up rows of 64 h columns, interleaved 16 by
 * 16 per wave; W2: 128 output rows) and 128-deep K chunk c, the 4 waves' 32 rows
 * each are stored as [g][nt][c][wave][load][lane][16 bytes], so each wave load
 * reads 1 KiB of contiguous memory and each workgroup streams one sequential
 * region (the row-major layout makes a workgroup read 128 rows in 256-byte
 * pieces, which MI355X HBM serves at about two thirds of the rate).
 *
 * w13 [G, 2I, H] -> w13_packed, w2 [G, H, I] -> w2_packed, same byte sizes,
 * w_dt MOE_BF16 or MOE_FP8_E4M3 (fp8 scales keep their layout). Either pair may
 * be NULL to skip it. Not in place. H and I multiples of 128.
 */
moe_status_t moe_pack_weights(int n_groups, int hidden, int inter, moe_dtype_t w_dt, const void* w13, const void* w2,
                              void* w13_packed, void* w2_packed, hipStream_t stream);

/* ------------------------------------------------------------------ combine
 * Undo the dispatch permutation and take the router-weighted sum (lehuy.net
 * page, section Throughput > Combine; AWS EFA page, section MoE all-to-all
 * over EFA: the combine returns each token's weighted average), summed at the
 * sender over this GPU's experts (AWS EFA page, section Evaluation). For a
 * token t with a kept entry, or self_lo <= t < self_hi when shared_y is given:
 *   out[t] = sum over k ascending with row_of[t*K+k] in [0, n_rows) of
 *            topk_w[t*K+k] * ye[row] + [t in self] shared_y[t - self_lo]
 * accumulated in fp32 and rounded once to dt. Other rows of out are not written.
 *
 * ye [n_rows, hidden] (dt), topk_w [N, K] float32, shared_y
 * [self_hi - self_lo, hidden] (dt) or NULL, out [N, hidden] (dt).
 */
moe_status_t moe_combine(const void* ye, moe_dtype_t dt, int64_t n_rows, const int32_t* row_of,
                         const float* topk_w, int n_tokens, int top_k, int hidden, const void* shared_y,
                         int self_lo, int self_hi, void* out, hipStream_t stream);

/* moe_combine for the tokens the down projection's scatter (moe_scatter_t,
 * same n_rows, self_lo and self_hi) did not write: those with two or more
 * kept entries, and those in [self_lo, self_hi) with a shared_y row. Tokens
 * with exactly one kept entry outside that range are left as they are. Same
 * arguments and errors as moe_combine. */
moe_status_t moe_combine_multi(const void* ye, moe_dtype_t dt, int64_t n_rows, const int32_t* row_of,
                               const float* topk_w, int n_tokens, int top_k, int hidden, const void* shared_y,
                               int self_lo, int self_hi, void* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
