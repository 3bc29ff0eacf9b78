/*
 * moe_shuffle.h -- C ABI of the MI355X (gfx950) MoE token dispatch/combine
 * library (libmoe_shuffle.so).
 *
 * The path: route and shuffle (moe_shuffle), dispatch (moe_gather_scale or its
 * FP8 rowwise form), expert GEMMs (not here), combine (moe_scatter_add) or the
 * fused MoE tail (moe_finalize_rmsnorm).
 *
 * Sources (web pages, cited by title and section):
 *   [GS] "mslk/moe/gather_scatter.py" (mslk-cuda-nightly wheel)
 *   [LY] "mslk/moe/layers.py" (same wheel)
 *   [K3] "vllm ... kimi_k3 ... allreduce_rmsnorm_reduce_scatter_early_exit"
 *   [MH] "vllm ... deepseek_v41 ... all_reduce_mhc"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer except where marked "host".
 *    bf16 tensors are uint16_t bit patterns; FP8 is OCP E4M3FN (uint8_t);
 *    MXFP8 scales are UE8M0 exponent bytes (uint8_t). All tensors are
 *    row-major and dense unless a stride argument says otherwise.
 *  - `stream` is a hipStream_t passed as void* (NULL: the null stream). Work
 *    is enqueued on it and the call returns; nothing synchronises the host and
 *    the library never reads device memory from the host. Device-side counts
 *    (valid_token_count, valid_rows) are read by the kernels.
 *  - The caller owns all memory. The library allocates nothing, keeps no
 *    pointer after a call returns and holds no state; calls are reentrant.
 *    Calls that share output or workspace memory must be ordered by the
 *    caller (same stream, or events). The one exception is
 *    moe_shuffle_noalloc, whose workspace is a static device array of the
 *    library (see there).
 *  - Errors: all argument checks run on the host before any launch. On a
 *    failed check nothing is enqueued and the status says why
 *    (moe_last_error() gives a message for the calling thread):
 *      MOE_ERR_INVALID_ARG  NULL required pointer, negative or too large size,
 *                           misaligned pointer, K outside [1, E], D not a
 *                           multiple of the vector width (8 bf16 elements;
 *                           32 for MXFP8 output)
 *      MOE_ERR_UNSUPPORTED  a size beyond what the kernels are built for
 *                           (E > 1024, K > 64)
 *      MOE_ERR_WORKSPACE    workspace NULL or smaller than *_workspace_bytes
 *      MOE_ERR_HIP          a HIP launch error (hipGetLastError after launch)
 *    A call with nothing to do (T == 0, a == 0 or D == 0) returns MOE_OK and
 *    enqueues nothing, except moe_shuffle, which still writes counts (zeros).
 *  - Device-side values are preconditions (as on the pages): indices must be
 *    in range. The kernels range-check every index they address memory with
 *    and skip an out-of-range row rather than fault; what they write for it is
 *    unspecified. Device-side counts are clamped to [0, T] / [0, a].
 *  - Row buffers (x, out, in_tokens, y, shared, gamma, codes) must be 16-byte
 *    aligned; index and score buffers 4-byte aligned.
 */
#ifndef MOE_SHUFFLE_H
#define MOE_SHUFFLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point is exported from the shared library. */
#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

typedef uint16_t moe_bf16_t; /* bfloat16 bit pattern */

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_WORKSPACE = 3,
    MOE_ERR_HIP = 4
} moe_status_t;

/* Version of this ABI (bumped on any signature change). */
#define MOE_ABI_VERSION 3
MOE_API int moe_abi_version(void);

/* Static name of a status code. */
MOE_API const char *moe_status_str(moe_status_t status);

/* Message of the last failed call on the calling thread ("" if none). The
 * returned string is thread-local and valid until the next call. */
MOE_API const char *moe_last_error(void);

/* ------------------------------------------------------------------------
 * moe_shuffle -- top-k routing and the stable counting sort of
 * (token, expert) pairs by expert.
 *
 * [LY] MetaShufflingMoE._route hands the router scores to the shuffle, which
 * returns per-expert token counts plus the expert and token index of every
 * routed row, grouped by expert; the grouped GEMMs and [GS]
 * gather_scale_dense_tokens then read rows in that order. [LY]
 * BaselineMoE._forward defines the routing as the K largest scores per token.
 *
 * For each token t < vtc (vtc = *valid_token_count clamped to [0, T], or T
 * when NULL) the K experts with the largest scores are selected; slot k is
 * the k-th largest; equal scores go to the lower expert id (+0 and -0 are
 * equal). Scores must not be NaN.
 *   counts[e] (e < E)  number of selected pairs of expert e
 *   counts[E]          V = vtc * K, the number of valid rows (the row bound
 *                      that moe_gather_scale / moe_scatter_add take)
 *   rows [0, V)        the valid pairs sorted by (expert, token): a stable
 *                      sort, so within an expert tokens ascend
 *   rows [V, T*K)      the pairs of tokens t >= vtc in (t, k) order, with
 *                      token_indices = t and expert_indices = -1
 *   row_of_pair[t*K+k] row of pair (t, k); -1 for t >= vtc. It is the inverse
 *                      of token_indices on the valid rows, and is what the
 *                      finalize takes as its permuted-row map.
 * The result is deterministic (no order depends on timing).
 *
 * scores           [T, E] fp32, element (t, e) at scores[t*stride_t + e*stride_e]
 *                  (strides in elements, >= 0)
 * valid_token_count  nullable device int32 scalar
 * counts           [E+1] int32 out
 * expert_indices, token_indices  [T*K] int32 out
 * row_of_pair      [T*K] int32 out, nullable
 * workspace        >= moe_shuffle_workspace_bytes(T, E, K) bytes, 256-byte
 *                  aligned, contents ignored on entry and undefined after
 * Limits: 1 <= E <= 1024, 1 <= K <= min(E, 64), T*K < 2^31.
 * ---------------------------------------------------------------------- */
MOE_API size_t moe_shuffle_workspace_bytes(int32_t T, int32_t E, int32_t K);
MOE_API moe_status_t moe_shuffle(const float *scores, int64_t stride_t, int64_t stride_e,
                         int32_t T, int32_t E, int32_t K,
                         const int32_t *valid_token_count, int32_t *counts,
                         int32_t *expert_indices, int32_t *token_indices,
                         int32_t *row_of_pair, void *workspace,
                         size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * moe_shuffle_noalloc -- moe_shuffle without a workspace argument, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * serving loops that must not call the allocator, harnesses that forbid it.
 *
 * Same arguments, results and checks as moe_shuffle, and the same kernels.
 * The workspace is instead a static device array of the library,
 * MOE_NOALLOC_SCRATCH_BYTES bytes, of which each GPU the library runs on
 * holds its own copy until the process ends. The call allocates nothing and
 * calls no allocating routine. Its kernels write every scratch byte they read
 * before reading it, so nothing needs clearing between calls.
 *
 * Errors, beyond moe_shuffle's:
 *   MOE_ERR_WORKSPACE    moe_shuffle_workspace_bytes(T, E, K) exceeds
 *                        MOE_NOALLOC_SCRATCH_BYTES (e.g. T = 8192, E = 256,
 *                        K = 8 needs 512 KiB)
 *   MOE_ERR_INVALID_ARG  `stream` belongs to another device than the
 *                        current one (the scratch address is per device)
 *   MOE_ERR_HIP          the scratch address could not be obtained
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one GPU (different streams, or threads without ordering) race and give
 * undefined results. Order them on one stream.
 * ---------------------------------------------------------------------- */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
MOE_API moe_status_t moe_shuffle_noalloc(const float *scores, int64_t stride_t,
                                 int64_t stride_e, int32_t T, int32_t E, int32_t K,
                                 const int32_t *valid_token_count, int32_t *counts,
                                 int32_t *expert_indices, int32_t *token_indices,
                                 int32_t *row_of_pair, void *stream);

/* ------------------------------------------------------------------------
 * moe_gather_scale -- dispatch: gather token rows into expert order, scaled
 * by their router score.
 *
 * [GS] gather_scale_dense_tokens: for every row i < V (V = *valid_rows
 * clamped to [0, a], or a when NULL; the pages call it valid_token_count),
 *   t = token_indices[i], e = expert_indices[i],
 *   out[i, :] = bf16_rne( f32(x[t, :]) * scores[t*stride_t + e*stride_e] )
 * (one fp32 multiply per element). Rows i >= V are not written, nor rows
 * whose t or e is out of range.
 *
 * With a workspace (>= moe_gather_scale_workspace_bytes(T, a) bytes,
 * 256-byte aligned) the rows are visited token by token, so each row of x is
 * read from memory once: up to 1024 rows each token's rows are found
 * directly; beyond that through a list of each token's rows built in the
 * workspace first (one extra launch up to 4096 rows and tokens, two up to
 * 131072 rows, four beyond). With workspace == NULL, row by row (x re-read
 * once per row that uses it). The output is the same bit for bit. The
 * workspace is scratch: its contents on entry do not matter.
 *
 * x     [T, D] bf16;  out [a, D] bf16;  token_indices, expert_indices [a] int32
 * D % 8 == 0.
 * ---------------------------------------------------------------------- */
MOE_API size_t moe_gather_scale_workspace_bytes(int32_t T, int32_t a);
MOE_API moe_status_t moe_gather_scale(const moe_bf16_t *x, int32_t T, int32_t D,
                              const int32_t *token_indices,
                              const int32_t *expert_indices, int32_t a,
                              const float *scores, int64_t stride_t,
                              int64_t stride_e, int32_t E,
                              const int32_t *valid_rows, moe_bf16_t *out,
                              void *workspace, size_t workspace_bytes, void *stream);

/* moe_gather_scale_by_token -- the same output as moe_gather_scale, visiting
 * the rows token by token through the inverse map row_of_pair ([T, K] int32,
 * as moe_shuffle writes it), so each token row of x is read from memory once
 * and written to its K rows. Pairs with row < 0 or row >= V are skipped.
 * Precondition: row_of_pair is the inverse of token_indices on rows [0, V)
 * (it is, when both come from one moe_shuffle call); then the output equals
 * moe_gather_scale's bit for bit. */
MOE_API moe_status_t moe_gather_scale_by_token(const moe_bf16_t *x, int32_t T, int32_t D,
                                       const int32_t *row_of_pair, int32_t K,
                                       const int32_t *expert_indices, int32_t a,
                                       const float *scores, int64_t stride_t,
                                       int64_t stride_e, int32_t E,
                                       const int32_t *valid_rows,
                                       moe_bf16_t *out, void *stream);

/* ------------------------------------------------------------------------
 * moe_gather_scale_quant -- dispatch with FP8 (E4M3FN) rowwise quantisation.
 *
 * [GS] gather_scale_quant_dense_tokens and its FP8 rowwise kernel. For every
 * row i < V: v = f32(x[t, :]) * s (s as in moe_gather_scale);
 *   m = max_d |v_d|; m = clamp(m, EPS, *scale_ub) if scale_ub is given,
 *   else max(m, EPS), EPS = 1e-12;
 *   mult = 448 / m (correctly rounded);  out_scale[i] = 1 / mult;
 *   out_fp8[i, d] = e4m3_rne( clamp(v_d * mult, -448, 448) ).
 * Rows i >= V are not written (codes nor scale).
 *
 * scale_ub   nullable device fp32 scalar (the pages' CLAMP_MAX)
 * out_fp8    [a, D] uint8 E4M3FN codes, 16-byte aligned
 * out_scale  [a] fp32 dequantisation scale (value = code * out_scale)
 * D % 8 == 0.
 * ---------------------------------------------------------------------- */
MOE_API moe_status_t moe_gather_scale_quant(const moe_bf16_t *x, int32_t T, int32_t D,
                                    const int32_t *token_indices,
                                    const int32_t *expert_indices, int32_t a,
                                    const float *scores, int64_t stride_t,
                                    int64_t stride_e, int32_t E,
                                    const float *scale_ub,
                                    const int32_t *valid_rows, uint8_t *out_fp8,
                                    float *out_scale, void *stream);

/* ------------------------------------------------------------------------
 * moe_scatter_add -- combine: add expert output rows back into token order.
 *
 * [GS] scatter_add_dense_tokens adds every valid input row r < V into output
 * token token_indices[r]; [LY] _combine_outputs passes the shared-expert
 * output as the initial out. The pages add with atomics in no fixed order;
 * here the order is fixed and the result deterministic: for each token t,
 *   acc = f32(out[t, :]);  for each valid row r with token_indices[r] == t,
 *   in ascending r: acc += f32(in[r, :]);  out[t, :] = bf16_rne(acc).
 * Tokens with no valid row are not written.
 *
 * out_tokens [T, D] bf16 in/out;  in_tokens [a, D] bf16;  token_indices [a]
 * valid_rows nullable device int32 scalar (V, clamped to [0, a])
 * workspace  >= moe_scatter_add_workspace_bytes(T, a) bytes, 256-byte aligned
 * D % 8 == 0. Up to 1024 rows each token's rows are found directly (one
 * launch); beyond that a list of each token's rows is built in the workspace
 * first, and tokens routed to more than 64 valid rows take a slower
 * (quadratic in that count) ordering step. The result is the same.
 * ---------------------------------------------------------------------- */
MOE_API size_t moe_scatter_add_workspace_bytes(int32_t T, int32_t a);
MOE_API moe_status_t moe_scatter_add(moe_bf16_t *out_tokens, int32_t T,
                             const moe_bf16_t *in_tokens,
                             const int32_t *token_indices, int32_t a, int32_t D,
                             const int32_t *valid_rows, void *workspace,
                             size_t workspace_bytes, void *stream);

/* moe_scatter_add_by_token -- the same result as moe_scatter_add, reading each
 * token's rows from the inverse map row_of_pair ([T, K] int32, as moe_shuffle
 * writes it) instead of building it: no workspace, one launch. Rows < 0 or
 * >= V are skipped; the remaining rows of a token are added in ascending row
 * order. Precondition: row_of_pair is the inverse of token_indices on rows
 * [0, V); then the output equals moe_scatter_add's bit for bit. K <= 64. */
MOE_API moe_status_t moe_scatter_add_by_token(moe_bf16_t *out_tokens, int32_t T,
                                      const moe_bf16_t *in_tokens,
                                      const int32_t *row_of_pair, int32_t K,
                                      int32_t a, int32_t D,
                                      const int32_t *valid_rows, void *stream);

/* ------------------------------------------------------------------------
 * moe_scatter_add_padded -- the static-shape expert-parallel combine.
 *
 * [GS] scatter_add_padded_tokens, as [LY] _combine_outputs uses it after the
 * static (all-gather) exchange of _static_comm_forward. in_tokens is
 * [EP, T_K, D]: rank r's slab holds, at the row positions of the experts it
 * owns, those rows' expert outputs. token_counts [E] are the per-expert
 * counts of the shuffle (moe_shuffle's counts[0..E)); expert e's rows are
 * [off_e, off_e + counts[e]) with off_e the exclusive prefix of counts, and
 * are read from rank e / (E / EP). Each is added into
 * out_tokens[token_indices[row]] with moe_scatter_add's order and rounding:
 * per token, the initial value, then its rows in ascending row index, in
 * fp32, rounded once to bf16; tokens with no row are not written.
 *
 * in_tokens [EP, T_K, D] bf16; token_counts [E] int32 (device; the row total
 * is clamped to T_K); token_indices [T_K] int32; out_tokens [T, D] bf16
 * in/out. E % EP == 0, 1 <= E <= 1024, D % 8 == 0, EP * T_K < 2^31.
 * workspace >= moe_scatter_add_padded_workspace_bytes(T, T_K, E), 256-byte
 * aligned.
 * ---------------------------------------------------------------------- */
MOE_API size_t moe_scatter_add_padded_workspace_bytes(int32_t T, int32_t T_K, int32_t E);
MOE_API moe_status_t moe_scatter_add_padded(const moe_bf16_t *in_tokens, int32_t EP,
                                            int32_t T_K, const int32_t *token_counts,
                                            int32_t E, const int32_t *token_indices,
                                            moe_bf16_t *out_tokens, int32_t T, int32_t D,
                                            void *workspace, size_t workspace_bytes,
                                            void *stream);

/* moe_scatter_add_padded_by_token -- the same result as moe_scatter_add_padded,
 * reading each token's rows from the inverse map row_of_pair ([T, K] int32,
 * as moe_shuffle writes it) instead of building it from token_indices: no
 * workspace, one launch. Rows < 0 or >= V (V = the count total, clamped to
 * T_K) are skipped; the remaining rows of a token are added in ascending row
 * order, each read from the slab of the rank that owns its expert.
 * Precondition: row_of_pair is the inverse of token_indices on rows [0, V);
 * then the output equals moe_scatter_add_padded's bit for bit. K <= 64; the
 * other arguments and limits are moe_scatter_add_padded's. */
MOE_API moe_status_t moe_scatter_add_padded_by_token(const moe_bf16_t *in_tokens, int32_t EP,
                                                     int32_t T_K,
                                                     const int32_t *token_counts, int32_t E,
                                                     const int32_t *row_of_pair, int32_t K,
                                                     moe_bf16_t *out_tokens, int32_t T,
                                                     int32_t D, void *stream);

/* ------------------------------------------------------------------------
 * moe_combine_shuffling / moe_split_shuffling -- the expert-parallel
 * receive-side re-sort and its inverse.
 *
 * [LY] _dynamic_comm_forward and _static_comm_forward call combine_shuffling
 * on the rows received from EP ranks before the expert GEMMs and
 * split_shuffling on the GEMM output before sending it back; the source of
 * both is absent from the pages, and this is the reading of their use.
 * Rows are grouped by source rank, and inside a rank's chunk by expert
 * column c in [0, C): segment (r, c) holds counts[r*C + c] rows. Rank r's
 * chunk starts at row r * rank_stride, or right after rank r-1's chunk when
 * rank_stride < 0 (packed, the dynamic exchange; a fixed stride is the
 * static exchange's [EP, T, D] buffer).
 *   combine: out[0..total) = the segments of the local columns [c_lo, c_hi)
 *            in expert-major order (for each local column, ranks 0..EP-1);
 *            out_counts[l] = rows of column c_lo + l, out_counts[c_hi-c_lo]
 *            = total. Rows of out beyond total are not written.
 *   split:   the inverse: in[0..total) (expert-major) goes back to the
 *            (rank, column) positions in out; other rows of out are not
 *            written. out_counts (nullable) as for combine.
 * Rows are copied bit for bit. Rows whose position falls outside in_rows /
 * out_rows are skipped.
 *
 * in [in_rows, D] bf16, out [out_rows, D] bf16; counts [EP, C] int32
 * (device); out_counts [c_hi - c_lo + 1] int32. 1 <= EP <= 64,
 * (c_hi - c_lo) * EP <= 4096, 0 <= c_lo <= c_hi <= C, D % 8 == 0, rows and
 * EP * rank_stride < 2^31. workspace >=
 * moe_shuffling_workspace_bytes(EP, c_hi - c_lo, expert-major rows), where
 * the expert-major rows are out_rows for combine and in_rows for split.
 * ---------------------------------------------------------------------- */
MOE_API size_t moe_shuffling_workspace_bytes(int32_t EP, int32_t n_local, int64_t em_rows);
MOE_API moe_status_t moe_combine_shuffling(const moe_bf16_t *in, int64_t in_rows,
                                           moe_bf16_t *out, int64_t out_rows, int32_t D,
                                           const int32_t *counts, int32_t EP, int32_t C,
                                           int32_t c_lo, int32_t c_hi, int64_t rank_stride,
                                           int32_t *out_counts, void *workspace,
                                           size_t workspace_bytes, void *stream);
MOE_API moe_status_t moe_split_shuffling(const moe_bf16_t *in, int64_t in_rows,
                                         moe_bf16_t *out, int64_t out_rows, int32_t D,
                                         const int32_t *counts, int32_t EP, int32_t C,
                                         int32_t c_lo, int32_t c_hi, int64_t rank_stride,
                                         int32_t *out_counts, void *workspace,
                                         size_t workspace_bytes, void *stream);

/* ------------------------------------------------------------------------
 * moe_finalize_rmsnorm -- the MoE tail: weighted top-k reduction, shared
 * expert add, RMSNorm, optional MXFP8 output.
 *
 * [K3] routed role, top-k finalize; [MH] AllReduceMHC.finalize (top-k
 * reduction and shared-expert add folded into one pass, fp32 weights) and
 * _LamportMHCDeviceKernel (RMSNorm and MXFP8 of the bf16 output). On one GPU
 * the tensor-parallel all-reduce of the pages is the identity. Per token t:
 *   acc = 0; for k = 0..K-1 with r = row_of_pair[t*K+k] >= 0:
 *       acc = fma(expert_weights[t*K+k], f32(y[r, :]), acc)
 *   if shared: acc = acc + f32(shared[t, :]);   h = bf16_rne(acc)
 *   ss = sum_d f32(h_d)^2, each square in fp32 (flags bit 0: rounded to bf16
 *        first, the bf16-square mode of [K3]), accumulated in fp64 and
 *        rounded once to fp32: a square of a bf16 value has at most 16
 *        significant bits, so the fp64 sum is exact or within a few fp64
 *        ulps and its fp32 rounding does not depend on the summation order
 *        except for sums that close to an fp32 rounding midpoint
 *   inv = 1 / sqrt(ss / D + eps), correctly rounded from double
 *   out[t, d] = bf16_rne( (f32(h_d) * inv) * f32(gamma_d) )
 * MXFP8 (mx_codes and mx_scales both set; D % 32 == 0): for each 32-element
 * block j of out[t, :]: amax = max |out|; p = amax * fp32(1/448);
 *   byte = clamp(ceil(log2 p) + 127, 0, 254) (0 when p == 0);
 *   mx_codes[t, 32j+i] = e4m3_rne(clamp(out * 2^(127-byte), -448, 448));
 *   scale layout: row-major mx_scales[t*(D/32) + j], or with
 *   MOE_FINALIZE_MX_SWIZZLED the 128x4-tiled layout [MH] writes for MXFP8
 *   GEMMs (its index helper is absent from the pages; the reading here:
 *   128-row x 4-column tiles of 512 bytes in row-tile-major order, row m and
 *   column j of a tile at (m%32)*16 + ((m%128)/32)*4 + j%4), with the
 *   scales of the padding rows up to a multiple of 128 written as zero;
 *   D % 128 == 0. moe_mxfp8_scale_bytes gives the buffer size of either.
 *
 * y_permuted    [rows, D] bf16 unweighted expert outputs in permuted order
 * expert_weights [T, K] fp32, or bf16 with MOE_FINALIZE_BF16_WEIGHTS ([K3]
 *               reads bf16 weights and widens them exactly)
 * row_of_pair   [T, K] int32 (-1: slot not held; values must be < rows)
 * shared        [T, D] bf16, nullable;  gamma [D] bf16
 * out           [T, D] bf16;  mx_codes [T, D] uint8 (16-byte aligned) and
 *               mx_scales (moe_mxfp8_scale_bytes(T, D, flags) bytes): both
 *               NULL or both set
 * flags         MOE_FINALIZE_BF16_SQUARES | MOE_FINALIZE_BF16_WEIGHTS |
 *               MOE_FINALIZE_MX_SWIZZLED; other bits must be 0
 * D % 8 == 0, D <= 65536; K <= 64.
 * ---------------------------------------------------------------------- */
#define MOE_FINALIZE_BF16_SQUARES 1u
#define MOE_FINALIZE_BF16_WEIGHTS 2u
#define MOE_FINALIZE_MX_SWIZZLED 4u
MOE_API size_t moe_mxfp8_scale_bytes(int32_t M, int32_t D, uint32_t flags);
MOE_API moe_status_t moe_finalize_rmsnorm(const moe_bf16_t *y_permuted, int64_t rows,
                                  const void *expert_weights,
                                  const int32_t *row_of_pair,
                                  const moe_bf16_t *shared,
                                  const moe_bf16_t *gamma, float eps, int32_t T,
                                  int32_t K, int32_t D, uint32_t flags,
                                  moe_bf16_t *out, uint8_t *mx_codes,
                                  uint8_t *mx_scales, void *stream);

/* ------------------------------------------------------------------------
 * moe_finalize_mhc -- the MoE tail of a hyper-connection (mHC) layer: the
 * routed sum h of moe_finalize_rmsnorm, mixed into the hc residual streams,
 * and the normalised collapse of the mixed streams as the next layer input.
 * [MH] AllReduceMHC.finalize and _LamportMHCDeviceKernel: the consumer's
 * residual add becomes the mHC post-mix and pre-mix collapse, which the
 * unchanged RMSNorm normalises; on one GPU the all-reduce is the identity.
 * Per token t and element d (h as in moe_finalize_rmsnorm, bf16):
 *   for each target stream j = 0..hc-1:
 *     mixed = f32(h) * post[t, j]
 *     for each source stream s = 0..hc-1: mixed = fma(f32(residual[t, s, d]),
 *                                                      comb[t, s, j], mixed)
 *     residual_out[t, j, d] = bf16_rne(mixed)
 *     collapse = fma(f32(residual_out[t, j, d]), pre[t, j], collapse)
 *   prenorm = bf16_rne(collapse); out[t, :] = RMSNorm of prenorm with gamma
 *   and eps, and its optional MXFP8, exactly as moe_finalize_rmsnorm does
 *   for h (same flags). The pages write each "a + b * c" step of the mix and
 *   the collapse; here each is one fused multiply-add.
 * Residual only (pre == NULL; out, mx_codes and mx_scales must be NULL,
 * gamma is ignored): only residual_out is written, for a consumer that
 * collapses the streams itself.
 *
 * residual, residual_out [T, hc, D] bf16 (16-byte aligned; they must not
 * overlap); post [T, hc] fp32; comb [T, hc, hc] fp32 indexed [source,
 * target]; pre [T, hc] fp32 or NULL. Other arguments as for
 * moe_finalize_rmsnorm. 1 <= hc <= 4; D % 8 == 0, D <= 32768; K <= 64.
 * ---------------------------------------------------------------------- */
MOE_API moe_status_t moe_finalize_mhc(const moe_bf16_t *y_permuted, int64_t rows,
                                      const void *expert_weights, const int32_t *row_of_pair,
                                      const moe_bf16_t *shared, const moe_bf16_t *residual,
                                      const float *post, const float *comb, const float *pre,
                                      const moe_bf16_t *gamma, float eps, int32_t T, int32_t K,
                                      int32_t D, int32_t hc, uint32_t flags,
                                      moe_bf16_t *residual_out, moe_bf16_t *out,
                                      uint8_t *mx_codes, uint8_t *mx_scales, void *stream);

/* ------------------------------------------------------------------------
 * moe_convert_check -- the device conversions the kernels use, exposed so that
 * a caller (and the test suite) can compare them with a reference: for
 * i < n, bf16_out[i] = bf16_rne(in[i]) and e4m3_out[i] =
 * e4m3_rne(clamp(in[i], -448, 448)). Either output may be NULL.
 * ---------------------------------------------------------------------- */
MOE_API moe_status_t moe_convert_check(const float *in, int64_t n, moe_bf16_t *bf16_out,
                               uint8_t *e4m3_out, void *stream);

/* ------------------------------------------------------------------------
 * moe_launch_floor -- measurement aid: a kernel with moe_finalize_rmsnorm's
 * grid and workgroup shape for (T, D), T workgroups of
 * moe_launch_floor_threads(T, D) threads, that does
 *   kind 0  nothing (the cost of the launch itself), or
 *   kind 1  per thread i < n = T * threads: a = src[i]; b = src[a.x % n];
 *           dst[i] = b.x + b.y + b.z + b.w (two dependent 16-byte loads and a
 *           store: the two memory round trips a finalize token takes).
 * Timed beside the finalize they bound what it can reach when it is
 * latency-bound (few tokens). src: n 16-byte elements (4 x uint32); dst: n
 * int32. Both may be NULL for kind 0. T in [1, 2^20], D % 8 == 0 and
 * 8 <= D <= 65536.
 * ---------------------------------------------------------------------- */
MOE_API int32_t moe_launch_floor_threads(int32_t T, int32_t D);
MOE_API moe_status_t moe_launch_floor(int32_t kind, int32_t T, int32_t D, const void *src,
                              int32_t *dst, void *stream);

/* ------------------------------------------------------------------------
 * moe_stream_probe -- measurement aid: a plain contiguous stream with a
 * chosen read:write mix, units waves of R KiB read and W KiB written, every
 * access a nontemporal 16-byte one per lane. Layout 0 (blocked): wave u
 * reads the R KiB of src from byte u * R * 1024 and writes the W KiB of dst
 * from byte u * W * 1024. Layout 1 (interleaved): src is R streams and dst W
 * streams of units KiB each (stream r from byte r * units * 1024); wave u
 * reads KiB u of every source stream and writes KiB u of every destination
 * stream. Either way consecutive waves touch consecutive memory. Word j
 * (uint32) of the wave's w-th destination KiB is the wrapping sum over
 * r < R of word j of its r-th source KiB, xor w. Timed with a streaming
 * kernel's read and write bytes, it gives a reference rate for that mix on
 * this GPU (what a plain stream of the same bytes reaches), beside the HBM
 * peak.
 * layout 0 or 1; R and W in [1, 32]; units in [0, 2^31) (0: nothing is
 * launched). src holds at least units * R KiB, dst at least units * W KiB
 * (the caller's to guarantee: the call sees no sizes); both 16-byte
 * aligned, and the two ranges must not overlap (MOE_ERR_INVALID_ARG). Only
 * dst is written.
 * ---------------------------------------------------------------------- */
MOE_API moe_status_t moe_stream_probe(int32_t layout, int32_t R, int32_t W, int64_t units,
                                      const void *src, void *dst, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_SHUFFLE_H */
