/*
 * CPU oracle for the MoE dispatch/combine path.
 *
 * TEST INFRASTRUCTURE ONLY. This file is the slow, plain, single-threaded
 * statement of what each stage computes. Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load it; the product library
 * never does, and the two share no code, header, table or helper.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math (no FMA contraction,
 * no reassociation). Every float operation below is one IEEE-754 binary32
 * operation in round-to-nearest-even, except where fmaf() is written out.
 *
 * Sources (web pages; cited by page title and section):
 *   [GS]  "mslk/moe/gather_scatter.py" (mslk-cuda-nightly wheel): the
 *         gather_scale_dense_tokens, gather_scale_quant_dense_tokens and
 *         scatter_add_dense_tokens functions and their Triton kernels.
 *   [LY]  "mslk/moe/layers.py" (same wheel): MetaShufflingMoE._route,
 *         BaselineMoE._forward, MetaShufflingMoE._combine_outputs.
 *   [K3]  "vllm ... kimi_k3 ... allreduce_rmsnorm_reduce_scatter_early_exit":
 *         AllReduceRMSNormWithReduceScatterEarlyExit._token_device, routed role
 *         (top-k finalize reduction, RMSNorm).
 *   [MH]  "vllm ... deepseek_v41 ... all_reduce_mhc": AllReduceMHC.finalize and
 *         _LamportMHCDeviceKernel (RMSNorm, MXFP8 output).
 *
 * Parity status: every function here is pinned by a CPU test against
 * something other than itself (brute force, torch library casts/routines,
 * exact rational arithmetic, closed forms, invariants). Parity unpinned, as
 * readings of steps the pages call but do not print: the scale of an
 * all-zero row in gather_scale_quant (an EPS constant), the round-up
 * direction of the UE8M0 scale, the 128x4 tile order of the swizzled
 * scales (beyond its innermost axis: the pages' padding stores fix that a
 * row's 4 columns of a tile are 4 contiguous, 4-aligned bytes), and the EP
 * re-sort layout; each is pinned against a restatement of its reading, not
 * against the pages.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD 1

/* Largest finite OCP E4M3FN magnitude: 1.75 * 2^8. */
#define E4M3_MAX 448.0f
/* Row-max floor of the FP8 rowwise quantiser. The pages take it from a helper
 * whose source is absent; 1e-12 is this oracle's reading. */
#define ROWWISE_EPS 1e-12f

/* ------------------------------------------------------------------------ */
/* Number formats, written from their definitions.                           */
/* ------------------------------------------------------------------------ */

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* bfloat16 is the upper half of a binary32. Widening is exact. */
float orc_bf16_to_f32(uint16_t h) { return bits_f32((uint32_t)h << 16); }

/* binary32 -> bfloat16, round to nearest, ties to even. The dropped low 16
 * bits decide: above half rounds up, below half truncates, exactly half rounds
 * to the even result. NaN stays NaN (quiet bit set). Overflow rounds to inf. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u = f32_bits(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16;
    uint32_t rest = u & 0xFFFFu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u)))
        keep += 1u; /* a carry into the exponent is the correct result */
    return (uint16_t)keep;
}

/* Round a non-negative double to the nearest integer, ties to even. */
static double round_half_even(double v)
{
    double fl = floor(v);
    double diff = v - fl;
    if (diff > 0.5) return fl + 1.0;
    if (diff < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* binary32 -> OCP FP8 E4M3FN (1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; no infinities; S.1111.111 is NaN; largest finite 448 = 0x7E).
 * Round to nearest even; magnitudes that round above 448 saturate to 448
 * ("satfinite"). NaN maps to 0x7F. The sign of zero is kept (-0 -> 0x80). */
uint8_t orc_f32_to_e4m3(float f)
{
    if (isnan(f)) return 0x7F;
    uint8_t sign = signbit(f) ? 0x80 : 0x00;
    if (isinf(f)) return (uint8_t)(sign | 0x7E);
    double a = fabs((double)f);
    uint8_t mag;
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: value = m * 2^-9, m in 0..7; m == 8 is the
         * smallest normal 2^-6, whose code 0x08 is also m. */
        double m = round_half_even(a * 512.0);
        mag = (uint8_t)m;
    } else {
        int ex;
        double fr = frexp(a, &ex); /* a = fr * 2^ex, fr in [0.5, 1) */
        int e_unb = ex - 1;        /* a = (2 fr) * 2^e_unb, 2 fr in [1, 2) */
        double m = round_half_even((2.0 * fr - 1.0) * 8.0);
        if (m == 8.0) { m = 0.0; e_unb += 1; }
        int biased = e_unb + 7;
        if (biased > 15 || (biased == 15 && m > 6.0)) {
            mag = 0x7E; /* satfinite */
        } else {
            mag = (uint8_t)((biased << 3) | (int)m);
        }
    }
    return (uint8_t)(sign | mag);
}

/* OCP E4M3FN code -> binary32 (exact). */
float orc_e4m3_to_f32(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (float)(s ? -v : v);
}

/* UE8M0 shared scale of one MXFP8 block, from the block's absolute maximum.
 * [MH] _LamportMHCDeviceKernel, MXFP8 quantize: the block max is multiplied by
 * the reciprocal of the E4M3 maximum (one binary32 multiply by the binary32
 * constant 1/448) and turned into an 8-bit power-of-two exponent. Reading: the
 * exponent rounds up (ceil of log2), so the scaled block max never exceeds 448;
 * a zero product gives byte 0; the byte is clamped to [0, 254] (255 is NaN). */
uint8_t orc_ue8m0_from_amax(float amax)
{
    const float inv_max = 1.0f / E4M3_MAX;
    float p = amax * inv_max;
    if (p == 0.0f) return 0;
    int ex;
    float fr = frexpf(p, &ex); /* p = fr * 2^ex, fr in [0.5, 1) */
    int ceil_log2 = (fr == 0.5f) ? ex - 1 : ex;
    int byte = ceil_log2 + 127;
    if (byte < 0) byte = 0;
    if (byte > 254) byte = 254;
    return (uint8_t)byte;
}

/* ------------------------------------------------------------------------ */
/* Routing: top-k selection and the stable counting-sort shuffle.            */
/* ------------------------------------------------------------------------ */

static int clamp_count(long long v, long long hi)
{
    if (v < 0) return 0;
    if (v > hi) return (int)hi;
    return (int)v;
}

/* Top-k of one token's scores. [LY] BaselineMoE._forward takes the K largest
 * router scores per token; MetaShufflingMoE._route hands the raw scores to the
 * shuffle. Reading: slots run by score descending; equal scores go to the
 * lower expert id (IEEE equality, so -0 and +0 tie). Scores must not be NaN.
 * Selection sort: K passes, each taking the best not-yet-taken expert. */
static void topk_row(const float *scores, long long st, long long se, int t,
                     int E, int K, int *sel, unsigned char *taken)
{
    memset(taken, 0, (size_t)E);
    for (int k = 0; k < K; ++k) {
        int best = -1;
        float best_s = 0.0f;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            float s = scores[(long long)t * st + (long long)e * se];
            if (best < 0 || s > best_s) { best = e; best_s = s; }
        }
        taken[best] = 1;
        sel[k] = best;
    }
}

int orc_topk(const float *scores, long long st, long long se, int T, int E,
             int K, int *sel /* [T*K] */)
{
    if (T < 0 || E < 1 || K < 1 || K > E) return ORC_BAD;
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    for (int t = 0; t < T; ++t)
        topk_row(scores, st, se, t, E, K, sel + (long long)t * K, taken);
    free(taken);
    return ORC_OK;
}

/* The shuffle: a stable counting sort of the (token, expert) pairs of the
 * first vtc tokens by expert. [LY] MetaShufflingMoE._route calls the shuffle
 * on the router scores and keeps the first E counts; the grouped GEMM reads
 * rows expert by expert; [GS] gather_scale_dense_tokens then reads
 * token_indices / expert_indices row by row.
 *   counts[e]  number of valid pairs routed to e; counts[E] = vtc*K (all
 *              valid rows; the row bound that gather/scatter take).
 *   rows [0, V) are the valid pairs ordered by (expert, token), V = vtc*K.
 *   rows [V, T*K) hold the pairs of tokens t >= vtc in (t, k) order, with
 *              token_indices = t and expert_indices = -1.
 *   row_of_pair[t*K+k] is the row of pair (t, k), -1 for t >= vtc.
 * Without a valid count (has_vtc == 0) all T tokens are valid; a given count
 * is clamped to [0, T]. */
int orc_shuffle(const float *scores, long long st, long long se, int T, int E,
                int K, int has_vtc, long long vtc_in, int *counts /* [E+1] */,
                int *expert_indices, int *token_indices, int *row_of_pair)
{
    if (T < 0 || E < 1 || K < 1 || K > E) return ORC_BAD;
    int vtc = has_vtc ? clamp_count(vtc_in, T) : T;
    long long a = (long long)T * K;
    int *sel = (int *)malloc(sizeof(int) * (size_t)(a > 0 ? a : 1));
    unsigned char *taken = (unsigned char *)malloc((size_t)E);
    for (int t = 0; t < vtc; ++t)
        topk_row(scores, st, se, t, E, K, sel + (long long)t * K, taken);

    /* 1. histogram */
    for (int e = 0; e <= E; ++e) counts[e] = 0;
    for (int t = 0; t < vtc; ++t)
        for (int k = 0; k < K; ++k) counts[sel[(long long)t * K + k]] += 1;
    /* 2. exclusive scan */
    long long *next = (long long *)malloc(sizeof(long long) * (size_t)E);
    long long run = 0;
    for (int e = 0; e < E; ++e) { next[e] = run; run += counts[e]; }
    counts[E] = (int)run;
    /* 3. stable placement: tokens visited in ascending order */
    for (int t = 0; t < vtc; ++t) {
        for (int k = 0; k < K; ++k) {
            int e = sel[(long long)t * K + k];
            long long r = next[e]++;
            token_indices[r] = t;
            expert_indices[r] = e;
            if (row_of_pair) row_of_pair[(long long)t * K + k] = (int)r;
        }
    }
    /* 4. tail: pairs of the invalid tokens, in (t, k) order */
    for (int t = vtc; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            long long r = run + (long long)(t - vtc) * K + k;
            token_indices[r] = t;
            expert_indices[r] = -1;
            if (row_of_pair) row_of_pair[(long long)t * K + k] = -1;
        }
    }
    free(next);
    free(taken);
    free(sel);
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Dispatch: gather and scale.                                               */
/* ------------------------------------------------------------------------ */

/* [GS] gather_scale_dense_tokens and its kernel: output row i copies token
 * token_indices[i] scaled by its score scores[t, expert_indices[i]] (product
 * taken in fp32, stored in x's dtype), for rows below the valid bound only;
 * other rows are left as they were. Without a bound (has_valid == 0) all a
 * rows are valid; a given bound is clamped to [0, a] (as everywhere below). */
int orc_gather_scale(const uint16_t *x, int T, int D, const int *token_indices,
                     const int *expert_indices, int a, const float *scores,
                     long long st, long long se, int E, int has_valid,
                     long long valid_rows, uint16_t *out /* [a*D] */)
{
    if (T < 0 || D < 0 || a < 0 || E < 1) return ORC_BAD;
    int V = has_valid ? clamp_count(valid_rows, a) : a;
    for (int i = 0; i < V; ++i) {
        int t = token_indices[i], e = expert_indices[i];
        if (t < 0 || t >= T || e < 0 || e >= E) return ORC_BAD;
        float s = scores[(long long)t * st + (long long)e * se];
        for (int d = 0; d < D; ++d) {
            float v = orc_bf16_to_f32(x[(long long)t * D + d]) * s;
            out[(long long)i * D + d] = orc_f32_to_bf16(v);
        }
    }
    return ORC_OK;
}

/* [GS] gather_scale_quant_dense_tokens and its FP8 rowwise kernel. Per valid
 * row: v = x * s in fp32; m = max |v|; m is clamped to [EPS, ub] when an upper
 * bound is given, else floored at EPS; the quantisation multiplier is 448 / m;
 * the stored scale is its reciprocal; each element is (x * s) * multiplier,
 * clamped to [-448, 448] and converted to E4M3. scale_ub may be NULL. */
int orc_gather_scale_quant(const uint16_t *x, int T, int D,
                           const int *token_indices, const int *expert_indices,
                           int a, const float *scores, long long st,
                           long long se, int E, const float *scale_ub,
                           int has_valid, long long valid_rows,
                           uint8_t *out_fp8 /* [a*D] */,
                           float *out_scale /* [a] */)
{
    if (T < 0 || D < 0 || a < 0 || E < 1) return ORC_BAD;
    int V = has_valid ? clamp_count(valid_rows, a) : a;
    for (int i = 0; i < V; ++i) {
        int t = token_indices[i], e = expert_indices[i];
        if (t < 0 || t >= T || e < 0 || e >= E) return ORC_BAD;
        float s = scores[(long long)t * st + (long long)e * se];
        const uint16_t *xr = x + (long long)t * D;
        float m = 0.0f;
        for (int d = 0; d < D; ++d) {
            float v = orc_bf16_to_f32(xr[d]) * s;
            float av = fabsf(v);
            if (av > m) m = av;
        }
        if (scale_ub) {
            if (m < ROWWISE_EPS) m = ROWWISE_EPS;
            if (m > *scale_ub) m = *scale_ub;
        } else if (m < ROWWISE_EPS) {
            m = ROWWISE_EPS;
        }
        float mult = E4M3_MAX / m;
        out_scale[i] = 1.0f / mult;
        for (int d = 0; d < D; ++d) {
            float v = orc_bf16_to_f32(xr[d]) * s;
            float q = v * mult;
            if (q > E4M3_MAX) q = E4M3_MAX;
            if (q < -E4M3_MAX) q = -E4M3_MAX;
            out_fp8[(long long)i * D + d] = orc_f32_to_e4m3(q);
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Combine: scatter-add expert outputs back to token order.                  */
/* ------------------------------------------------------------------------ */

/* [GS] scatter_add_dense_tokens: every valid input row r is added into output
 * token token_indices[r]. [LY] _combine_outputs passes the shared-expert output
 * as the initial out. The pages add with atomics in unspecified order; this
 * oracle fixes the order: per token, start from the initial value in fp32 and
 * add its rows in ascending row index, then round once to bf16. A token with
 * no valid row is left untouched. */
int orc_scatter_add(uint16_t *out /* [T*D] in/out */, int T,
                    const uint16_t *in /* [a*D] */, const int *token_indices,
                    int a, int D, int has_valid, long long valid_rows)
{
    if (T < 0 || D < 0 || a < 0) return ORC_BAD;
    int V = has_valid ? clamp_count(valid_rows, a) : a;
    /* bucket the valid rows by token, keeping ascending row order */
    int *cnt = (int *)calloc((size_t)T + 1, sizeof(int));
    for (int r = 0; r < V; ++r) {
        int t = token_indices[r];
        if (t < 0 || t >= T) { free(cnt); return ORC_BAD; }
        cnt[t + 1] += 1;
    }
    for (int t = 0; t < T; ++t) cnt[t + 1] += cnt[t];
    int *fill = (int *)malloc(sizeof(int) * (size_t)(T > 0 ? T : 1));
    int *rows = (int *)malloc(sizeof(int) * (size_t)(V > 0 ? V : 1));
    for (int t = 0; t < T; ++t) fill[t] = cnt[t];
    for (int r = 0; r < V; ++r) rows[fill[token_indices[r]]++] = r;
    float *acc = (float *)malloc(sizeof(float) * (size_t)(D > 0 ? D : 1));
    for (int t = 0; t < T; ++t) {
        if (cnt[t + 1] == cnt[t]) continue;
        uint16_t *o = out + (long long)t * D;
        for (int d = 0; d < D; ++d) acc[d] = orc_bf16_to_f32(o[d]);
        for (int j = cnt[t]; j < cnt[t + 1]; ++j) {
            const uint16_t *src = in + (long long)rows[j] * D;
            for (int d = 0; d < D; ++d) acc[d] = acc[d] + orc_bf16_to_f32(src[d]);
        }
        for (int d = 0; d < D; ++d) o[d] = orc_f32_to_bf16(acc[d]);
    }
    free(acc);
    free(rows);
    free(fill);
    free(cnt);
    return ORC_OK;
}

/* [GS] scatter_add_padded_tokens: the static-shape expert-parallel combine.
 * in is [EP, T_K, D]: rank r's slab holds, at the row positions of the
 * experts it owns, the outputs of those rows. counts [E] are the per-expert
 * row counts of the shuffle; the rows of expert e are [off_e, off_e +
 * counts[e]) with off_e the exclusive prefix of counts, and they come from
 * rank e / (E / EP). Each such row is added into out[token_indices[row]].
 * Same fixed order as orc_scatter_add: per token, the initial value then
 * its rows in ascending row index, fp32, one bf16 rounding; tokens with no
 * row are not written. E % EP == 0 and sum(counts) <= T_K are required. */
int orc_scatter_add_padded(uint16_t *out /* [T*D] in/out */, int T,
                           const uint16_t *in /* [EP*T_K*D] */, int EP, int T_K,
                           const int *counts /* [E] */, int E,
                           const int *token_indices /* [T_K] */, int D)
{
    if (T < 0 || D < 0 || EP < 1 || E < 1 || E % EP != 0 || T_K < 0) return ORC_BAD;
    long long V = 0;
    for (int e = 0; e < E; ++e) {
        if (counts[e] < 0) return ORC_BAD;
        V += counts[e];
    }
    if (V > T_K) return ORC_BAD;
    int *rank_of_row = (int *)malloc(sizeof(int) * (size_t)(V > 0 ? V : 1));
    long long off = 0;
    for (int e = 0; e < E; ++e) {
        for (int i = 0; i < counts[e]; ++i) rank_of_row[off + i] = e / (E / EP);
        off += counts[e];
    }
    /* bucket rows by token in ascending row order */
    int *cnt = (int *)calloc((size_t)T + 1, sizeof(int));
    for (long long r = 0; r < V; ++r) {
        int t = token_indices[r];
        if (t < 0 || t >= T) { free(cnt); free(rank_of_row); return ORC_BAD; }
        cnt[t + 1] += 1;
    }
    for (int t = 0; t < T; ++t) cnt[t + 1] += cnt[t];
    int *fill = (int *)malloc(sizeof(int) * (size_t)(T > 0 ? T : 1));
    int *rows = (int *)malloc(sizeof(int) * (size_t)(V > 0 ? V : 1));
    for (int t = 0; t < T; ++t) fill[t] = cnt[t];
    for (long long r = 0; r < V; ++r) rows[fill[token_indices[r]]++] = (int)r;
    float *acc = (float *)malloc(sizeof(float) * (size_t)(D > 0 ? D : 1));
    for (int t = 0; t < T; ++t) {
        if (cnt[t + 1] == cnt[t]) continue;
        uint16_t *o = out + (long long)t * D;
        for (int d = 0; d < D; ++d) acc[d] = orc_bf16_to_f32(o[d]);
        for (int j = cnt[t]; j < cnt[t + 1]; ++j) {
            int r = rows[j];
            const uint16_t *src =
                in + ((long long)rank_of_row[r] * T_K + r) * (long long)D;
            for (int d = 0; d < D; ++d) acc[d] = acc[d] + orc_bf16_to_f32(src[d]);
        }
        for (int d = 0; d < D; ++d) o[d] = orc_f32_to_bf16(acc[d]);
    }
    free(acc);
    free(rows);
    free(fill);
    free(cnt);
    free(rank_of_row);
    return ORC_OK;
}

/* [LY] combine_shuffling / split_shuffling (their source is absent; this is
 * the reading of how _dynamic_comm_forward and _static_comm_forward use
 * them). Rows arrive grouped by source rank, and inside a rank's chunk by
 * expert column c in [0, C): segment (r, c) holds counts[r*C + c] rows.
 * Rank r's chunk starts at r * rank_stride, or, with rank_stride < 0, right
 * after rank r-1's chunk (packed). combine gathers the columns of the local
 * expert range [c_lo, c_hi) into expert-major order -- for each local column,
 * the segments of ranks 0..EP-1 in turn -- and writes out_counts[l] = rows of
 * column c_lo + l and out_counts[c_hi - c_lo] = their total. split is the
 * inverse: rows in that expert-major order go back to their (rank, column)
 * positions. Rows are copied bit for bit. */
static int shuffling_table(const int *counts, int EP, int C, int c_lo, int c_hi,
                           long long rank_stride, long long *src_start,
                           long long *dst_start, long long *total)
{
    if (EP < 1 || C < 1 || c_lo < 0 || c_hi > C || c_lo > c_hi) return ORC_BAD;
    int nl = c_hi - c_lo;
    long long chunk = 0;  /* start of rank r's chunk */
    for (int r = 0; r < EP; ++r) {
        long long base = rank_stride >= 0 ? (long long)r * rank_stride : chunk;
        long long off = 0;
        for (int c = 0; c < C; ++c) {
            if (counts[r * C + c] < 0) return ORC_BAD;
            if (c >= c_lo && c < c_hi) src_start[(c - c_lo) * EP + r] = base + off;
            off += counts[r * C + c];
        }
        chunk = base + off;
    }
    long long run = 0;
    for (int l = 0; l < nl; ++l)
        for (int r = 0; r < EP; ++r) {
            dst_start[l * EP + r] = run;
            run += counts[r * C + c_lo + l];
        }
    *total = run;
    return ORC_OK;
}

int orc_shuffling(int inverse, const uint16_t *in, long long in_rows,
                  uint16_t *out, long long out_rows, int D, const int *counts,
                  int EP, int C, int c_lo, int c_hi, long long rank_stride,
                  int *out_counts /* [c_hi - c_lo + 1], may be NULL */)
{
    if (D < 0) return ORC_BAD;
    int nseg = (c_hi - c_lo) * EP;
    long long *src = (long long *)malloc(sizeof(long long) * (size_t)(nseg > 0 ? nseg : 1));
    long long *dst = (long long *)malloc(sizeof(long long) * (size_t)(nseg > 0 ? nseg : 1));
    long long total = 0;
    int rc = shuffling_table(counts, EP, C, c_lo, c_hi, rank_stride, src, dst, &total);
    for (int q = 0; rc == ORC_OK && q < nseg; ++q) {
        int r = q % EP, l = q / EP;
        long long len = counts[r * C + c_lo + l];
        for (long long j = 0; j < len; ++j) {
            long long a = src[q] + j, b = dst[q] + j; /* a: rank-major, b: expert-major */
            long long from = inverse ? b : a, to = inverse ? a : b;
            if (from >= in_rows || to >= out_rows) { rc = ORC_BAD; break; }
            memcpy(out + to * D, in + from * D, sizeof(uint16_t) * (size_t)D);
        }
    }
    if (rc == ORC_OK && out_counts) {
        for (int l = 0; l < c_hi - c_lo; ++l) {
            long long n = 0;
            for (int r = 0; r < EP; ++r) n += counts[r * C + c_lo + l];
            out_counts[l] = (int)n;
        }
        out_counts[c_hi - c_lo] = (int)total;
    }
    free(src);
    free(dst);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* MXFP8 of bf16 rows.                                                       */
/* ------------------------------------------------------------------------ */

/* [MH] _LamportMHCDeviceKernel, MXFP8 output: per 32-element block of a bf16
 * row, the UE8M0 byte of the block max (orc_ue8m0_from_amax), and codes
 * E4M3(o * 2^(127 - byte)) with saturation. Scales row-major [rows, D/32]. */
int orc_mxfp8_quantize(const uint16_t *o, int rows, int D, uint8_t *codes,
                       uint8_t *scales)
{
    if (rows < 0 || D < 0 || D % 32 != 0) return ORC_BAD;
    int nb = D / 32;
    for (int t = 0; t < rows; ++t) {
        const uint16_t *orow = o + (long long)t * D;
        for (int j = 0; j < nb; ++j) {
            float amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                float av = fabsf(orc_bf16_to_f32(orow[j * 32 + i]));
                if (av > amax) amax = av;
            }
            uint8_t byte = orc_ue8m0_from_amax(amax);
            scales[(long long)t * nb + j] = byte;
            float mult = ldexpf(1.0f, 127 - (int)byte);
            for (int i = 0; i < 32; ++i) {
                float v = orc_bf16_to_f32(orow[j * 32 + i]) * mult;
                codes[(long long)t * D + j * 32 + i] = orc_f32_to_e4m3(v);
            }
        }
    }
    return ORC_OK;
}

/* Byte size of an MXFP8 scale buffer for M rows of D elements: row-major
 * [M, D/32], or (swizzled) M rounded up to 128 times D/32 rounded up to 4
 * ([MH] mxfp8_scale_bytes; the layout below is this oracle's reading). */
long long orc_mxfp8_scale_bytes(int M, int D, int swizzled)
{
    long long cols = D / 32;
    if (!swizzled) return (long long)M * cols;
    long long mp = ((long long)M + 127) / 128 * 128;
    long long kp = (cols + 3) / 4 * 4;
    return mp * kp;
}

/* [MH] _LamportMHCDeviceKernel writes the MXFP8 scales "in the swizzled
 * 128x4 layout" of the MXFP8 GEMMs, zeroing the scales of the padding rows up
 * to a multiple of 128; the index helper is absent from the pages. Reading:
 * 128-row x 4-column tiles of 512 bytes in row-tile-major order; inside a
 * tile, row m and column k sit at (m % 32) * 16 + ((m % 128) / 32) * 4 +
 * (k % 4). Padding rows (and columns up to a multiple of 4) are zero. */
long long orc_mxfp8_swizzle_offset(int m, int k, int cols)
{
    long long kt_n = (cols + 3) / 4;
    long long tile = (long long)(m / 128) * kt_n + (k / 4);
    return tile * 512 + (m % 32) * 16 + ((m % 128) / 32) * 4 + (k % 4);
}

int orc_mxfp8_swizzle(const uint8_t *rowmajor /* [M, cols] */, int M, int cols,
                      uint8_t *out /* orc_mxfp8_scale_bytes(M, 32*cols, 1) */)
{
    if (M < 0 || cols < 0) return ORC_BAD;
    long long n = orc_mxfp8_scale_bytes(M, 32 * cols, 1);
    memset(out, 0, (size_t)n);
    for (int m = 0; m < M; ++m)
        for (int k = 0; k < cols; ++k)
            out[orc_mxfp8_swizzle_offset(m, k, cols)] = rowmajor[(long long)m * cols + k];
    return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Finalize: weighted top-k reduction + shared add + RMSNorm (+ MXFP8).      */
/* ------------------------------------------------------------------------ */

/* Per token t:
 *  [K3] routed role, top-k finalize: the fp32 sum over slots with a
 *       non-negative permuted row of weight * row value, in slot order.
 *       Written here as one fused multiply-add per slot.
 *  [MH] AllReduceMHC.finalize folds the shared-expert output into the same
 *       sum; reading: the shared value is added after the routed sum and the
 *       total is rounded once to bf16 (h).
 *  [MH] _LamportMHCDeviceKernel RMSNorm: sum of h^2 over the row (fp32
 *       squares; reading: the sum rounded once to fp32 from its exact value,
 *       see rmsnorm_row); inv = rsqrt(sum / D + eps); output
 *       bf16((h * inv) * gamma). With flags bit 0, each square is the
 *       bf16-rounded bf16 product, as in the [K3] default (non fp32_internal)
 *       mode. inv is the correctly rounded reciprocal square root (computed
 *       in double and rounded once).
 *  [MH] MXFP8 of the bf16 output, per 32-element block: UE8M0 byte from the
 *       block max (orc_ue8m0_from_amax); codes = E4M3(o * 2^(127 - byte)).
 *       Scales are stored row-major, [T, D/32]; with flags bit 2 in the
 *       swizzled 128x4 layout (orc_mxfp8_swizzle), D % 128 == 0.
 *  flags bit 1: the weights are bf16 (uint16 bits), widened exactly.
 * mx_codes and mx_scales are both NULL or both set; shared may be NULL. */
/* RMSNorm of one bf16 row ([MH] _LamportMHCDeviceKernel; [K3] routed role):
 * each square x^2 in fp32 (flags bit 0: rounded to bf16); their sum taken in
 * double, sequential in d, and rounded once to fp32 (ss); inv = correctly
 * rounded 1/sqrt(ss/D + eps); out = bf16((x * inv) * gamma).
 * Reading: the pages sum the squares in fp32 in an order set by their thread
 * layout, so the fp32 value depends on that order; the value every order
 * approximates is the exact sum. A square of a bf16 value has at most 16
 * significant bits, so the double sum is exact or off by a few double ulps,
 * and its rounding to fp32 is the fp32 nearest the exact sum unless the exact
 * sum lies that close to the midpoint of two fp32 values. */
static void rmsnorm_row(const uint16_t *x, const uint16_t *gamma, float eps, int D,
                        unsigned flags, uint16_t *out)
{
    double ss = 0.0;
    for (int d = 0; d < D; ++d) {
        float v = orc_bf16_to_f32(x[d]);
        float sq = v * v;
        if (flags & 1u) sq = orc_bf16_to_f32(orc_f32_to_bf16(sq));
        ss = ss + (double)sq;
    }
    float mean = (float)ss / (float)D;
    float arg = mean + eps;
    float inv = (float)(1.0 / sqrt((double)arg));
    for (int d = 0; d < D; ++d) {
        float v = orc_bf16_to_f32(x[d]) * inv;
        v = v * orc_bf16_to_f32(gamma[d]);
        out[d] = orc_f32_to_bf16(v);
    }
}

/* The routed sum of one token into h (bf16): fp32 fma over the held slots in
 * slot order, then + shared, one bf16 rounding. Returns ORC_BAD on a row
 * index >= rows. */
static int finalize_sum_row(const uint16_t *y, long long rows, const void *w,
                            const int *row_of_pair, const uint16_t *shared, int t,
                            int K, int D, unsigned flags, uint16_t *h)
{
    for (int k = 0; k < K; ++k)
        if (row_of_pair[(long long)t * K + k] >= rows) return ORC_BAD;
    for (int d = 0; d < D; ++d) {
        float acc = 0.0f;
        for (int k = 0; k < K; ++k) {
            long long r = row_of_pair[(long long)t * K + k];
            if (r < 0) continue;
            float wk = (flags & 2u)
                           ? orc_bf16_to_f32(((const uint16_t *)w)[(long long)t * K + k])
                           : ((const float *)w)[(long long)t * K + k];
            acc = fmaf(wk, orc_bf16_to_f32(y[r * D + d]), acc);
        }
        if (shared) acc = acc + orc_bf16_to_f32(shared[(long long)t * D + d]);
        h[d] = orc_f32_to_bf16(acc);
    }
    return ORC_OK;
}

int orc_finalize_rmsnorm(const uint16_t *y, long long rows, const void *w,
                         const int *row_of_pair, const uint16_t *shared,
                         const uint16_t *gamma, float eps, int T, int K, int D,
                         unsigned flags, uint16_t *out, uint8_t *mx_codes,
                         uint8_t *mx_scales)
{
    if (T < 0 || K < 1 || D < 1) return ORC_BAD;
    if ((mx_codes == NULL) != (mx_scales == NULL)) return ORC_BAD;
    if (mx_codes && D % 32 != 0) return ORC_BAD;
    int swizzled = (flags & 4u) != 0;
    if (swizzled && (!mx_codes || D % 128 != 0)) return ORC_BAD;
    uint8_t *rm_scales = NULL;
    if (swizzled) rm_scales = (uint8_t *)malloc((size_t)T * (size_t)(D / 32) + 1);
    uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)D);
    for (int t = 0; t < T; ++t) {
        if (finalize_sum_row(y, rows, w, row_of_pair, shared, t, K, D, flags, h) != ORC_OK) {
            free(h);
            if (rm_scales) free(rm_scales);
            return ORC_BAD;
        }
        uint16_t *o = out + (long long)t * D;
        rmsnorm_row(h, gamma, eps, D, flags, o);
        if (mx_codes)
            orc_mxfp8_quantize(o, 1, D, mx_codes + (long long)t * D,
                               (swizzled ? rm_scales : mx_scales) + (long long)t * (D / 32));
    }
    if (swizzled) {
        orc_mxfp8_swizzle(rm_scales, T, D / 32, mx_scales);
        free(rm_scales);
    }
    free(h);
    return ORC_OK;
}

/* [MH] AllReduceMHC.finalize with _LamportMHCDeviceKernel's mHC post-mix and
 * collapse, on one GPU (the tensor-parallel all-reduce is the identity, so
 * the reduced bf16 value is the finalize sum h of orc_finalize_rmsnorm).
 * Per token t and stream target j (hc streams):
 *   mixed = h * post[t][j]; for each source stream s in order:
 *       mixed = fma(residual[t][s], comb[t][s][j], mixed)
 *   residual_out[t][j] = bf16(mixed)
 *   collapse = fma(f32(residual_out[t][j]), pre[t][j], collapse)  (j in order)
 * then prenorm = bf16(collapse) is RMS-normalised into out (+ MXFP8) as in
 * orc_finalize_rmsnorm. comb is indexed [source][target]. Reading: each
 * "a + b * c" accumulation of the page is one fused multiply-add. With
 * pre == NULL only residual_out is written (gamma, out, MXFP8 unused). */
int orc_finalize_mhc(const uint16_t *y, long long rows, const void *w,
                     const int *row_of_pair, const uint16_t *shared,
                     const uint16_t *residual /* [T, hc, D] */, const float *post /* [T, hc] */,
                     const float *comb /* [T, hc, hc] */, const float *pre /* [T, hc] */,
                     const uint16_t *gamma, float eps, int T, int K, int D, int hc,
                     unsigned flags, uint16_t *residual_out /* [T, hc, D] */,
                     uint16_t *out, uint8_t *mx_codes, uint8_t *mx_scales)
{
    if (T < 0 || K < 1 || D < 1 || hc < 1) return ORC_BAD;
    if ((mx_codes == NULL) != (mx_scales == NULL)) return ORC_BAD;
    if (mx_codes && (D % 32 != 0 || pre == NULL)) return ORC_BAD;
    if (pre && (gamma == NULL || out == NULL)) return ORC_BAD;
    int swizzled = (flags & 4u) != 0;
    if (swizzled && (!mx_codes || D % 128 != 0)) return ORC_BAD;
    uint16_t *h = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)D);
    uint16_t *pn = (uint16_t *)malloc(sizeof(uint16_t) * (size_t)D);
    uint8_t *rm_scales = swizzled ? (uint8_t *)malloc((size_t)T * (size_t)(D / 32) + 1) : NULL;
    int rc = ORC_OK;
    for (int t = 0; t < T && rc == ORC_OK; ++t) {
        rc = finalize_sum_row(y, rows, w, row_of_pair, shared, t, K, D, flags, h);
        if (rc != ORC_OK) break;
        for (int d = 0; d < D; ++d) {
            float hv = orc_bf16_to_f32(h[d]);
            float collapse = 0.0f;
            for (int j = 0; j < hc; ++j) {
                float mixed = hv * post[(long long)t * hc + j];
                for (int src = 0; src < hc; ++src) {
                    float rv = orc_bf16_to_f32(residual[((long long)t * hc + src) * D + d]);
                    mixed = fmaf(rv, comb[((long long)t * hc + src) * hc + j], mixed);
                }
                uint16_t mb = orc_f32_to_bf16(mixed);
                residual_out[((long long)t * hc + j) * D + d] = mb;
                if (pre) collapse = fmaf(orc_bf16_to_f32(mb), pre[(long long)t * hc + j], collapse);
            }
            pn[d] = orc_f32_to_bf16(collapse);
        }
        if (!pre) continue;
        uint16_t *o = out + (long long)t * D;
        rmsnorm_row(pn, gamma, eps, D, flags, o);
        if (mx_codes)
            orc_mxfp8_quantize(o, 1, D, mx_codes + (long long)t * D,
                               (swizzled ? rm_scales : mx_scales) + (long long)t * (D / 32));
    }
    if (rc == ORC_OK && swizzled) orc_mxfp8_swizzle(rm_scales, T, D / 32, mx_scales);
    if (rm_scales) free(rm_scales);
    free(pn);
    free(h);
    return rc;
}

/* Element-wise helpers over arrays, exported so that the tests can run the
 * encoders exhaustively without a Python loop per element. */
void orc_f32_to_bf16_array(const float *in, uint16_t *out, long long n)
{
    for (long long i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(in[i]);
}
void orc_f32_to_e4m3_array(const float *in, uint8_t *out, long long n)
{
    for (long long i = 0; i < n; ++i) out[i] = orc_f32_to_e4m3(in[i]);
}
void orc_ue8m0_array(const float *amax, uint8_t *out, long long n)
{
    for (long long i = 0; i < n; ++i) out[i] = orc_ue8m0_from_amax(amax[i]);
}
