/*
 * A plain C consumer of libmoe_shuffle.so: it uses nothing but
 * include/moe_shuffle.h and the HIP runtime API, no Python and no torch.
 *
 *     c_abi_consumer IN OUT
 *
 * IN holds int32 T, E, K, D, then scores (T*E fp32), x (T*D bf16), y (T*K*D
 * bf16), out0 (T*D bf16), the finalize's routing weights w (T*K fp32),
 * shared (T*D bf16), gamma (D bf16) and eps (fp32). On the GPU the program
 * runs
 *   moe_shuffle;
 *   moe_gather_scale (token_indices, with a workspace) and
 *   moe_gather_scale_by_token, both into rows;
 *   moe_gather_scale_quant (token_indices, no upper clamp);
 *   moe_scatter_add (token_indices, with a workspace) and
 *   moe_scatter_add_by_token, each on its own copy of out0;
 *   moe_finalize_rmsnorm of y (in the shuffle's row order, through
 *   row_of_pair) with w, shared and gamma, with MXFP8 output when D % 32 == 0;
 * the valid row count staying on the device (counts[E]). OUT receives:
 * counts (E+1 int32), expert_indices, token_indices, row_of_pair (T*K int32
 * each), the two gathers' rows (T*K*D bf16 each), the FP8 codes (T*K*D) and
 * scales (T*K fp32), the two combines' outputs (T*D bf16 each), the finalize
 * output (T*D bf16), its MXFP8 codes (T*D) and row-major scales (T*D/32).
 * Every status is checked; on an error it prints the library's message and
 * exits with status 1.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "moe_shuffle.h"

#define HIP_OK(call)                                                              \
    do {                                                                          \
        hipError_t e_ = (call);                                                   \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));     \
            exit(1);                                                              \
        }                                                                         \
    } while (0)

#define MOE_OK(call)                                                              \
    do {                                                                          \
        moe_status_t s_ = (call);                                                 \
        if (s_ != MOE_OK) {                                                       \
            fprintf(stderr, "%s: %s: %s\n", #call, moe_status_str(s_),            \
                    moe_last_error());                                            \
            exit(1);                                                              \
        }                                                                         \
    } while (0)

static void *read_exact(FILE *f, size_t n) {
    void *p = malloc(n ? n : 1);
    if (!p || fread(p, 1, n, f) != n) {
        fprintf(stderr, "short input\n");
        exit(1);
    }
    return p;
}

static void *to_device(const void *h, size_t n) {
    void *d = NULL;
    HIP_OK(hipMalloc(&d, n ? n : 1));
    if (n) HIP_OK(hipMemcpy(d, h, n, hipMemcpyHostToDevice));
    return d;
}

static void write_back(FILE *f, const void *d, size_t n) {
    void *h = malloc(n ? n : 1);
    if (n) HIP_OK(hipMemcpy(h, d, n, hipMemcpyDeviceToHost));
    if (fwrite(h, 1, n, f) != n) {
        fprintf(stderr, "short write\n");
        exit(1);
    }
    free(h);
}

int main(int argc, char **argv) {
    if (argc != 3) {
        fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
        return 2;
    }
    FILE *fin = fopen(argv[1], "rb");
    if (!fin) {
        perror(argv[1]);
        return 1;
    }
    int32_t hdr[4];
    if (fread(hdr, sizeof(int32_t), 4, fin) != 4) {
        fprintf(stderr, "short header\n");
        return 1;
    }
    const int32_t T = hdr[0], E = hdr[1], K = hdr[2], D = hdr[3];
    if (T < 1 || E < 1 || K < 1 || K > E || D < 8 || D % 8) {
        fprintf(stderr, "bad sizes T=%d E=%d K=%d D=%d\n", T, E, K, D);
        return 1;
    }
    const size_t a = (size_t)T * (size_t)K;
    const size_t row_b = (size_t)D * 2;
    const int mx = D % 32 == 0;
    void *h_scores = read_exact(fin, (size_t)T * E * sizeof(float));
    void *h_x = read_exact(fin, (size_t)T * row_b);
    void *h_y = read_exact(fin, a * row_b);
    void *h_out = read_exact(fin, (size_t)T * row_b);
    void *h_w = read_exact(fin, a * sizeof(float));
    void *h_shared = read_exact(fin, (size_t)T * row_b);
    void *h_gamma = read_exact(fin, row_b);
    float eps;
    if (fread(&eps, sizeof eps, 1, fin) != 1) {
        fprintf(stderr, "short input\n");
        return 1;
    }
    fclose(fin);

    printf("moe_shuffle ABI %d: T=%d E=%d K=%d D=%d\n", moe_abi_version(), T, E, K, D);
    fflush(stdout);

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    float *scores = (float *)to_device(h_scores, (size_t)T * E * sizeof(float));
    moe_bf16_t *x = (moe_bf16_t *)to_device(h_x, (size_t)T * row_b);
    moe_bf16_t *y = (moe_bf16_t *)to_device(h_y, a * row_b);
    moe_bf16_t *out = (moe_bf16_t *)to_device(h_out, (size_t)T * row_b);
    moe_bf16_t *out_g = (moe_bf16_t *)to_device(h_out, (size_t)T * row_b);
    float *w = (float *)to_device(h_w, a * sizeof(float));
    moe_bf16_t *shared = (moe_bf16_t *)to_device(h_shared, (size_t)T * row_b);
    moe_bf16_t *gamma = (moe_bf16_t *)to_device(h_gamma, row_b);
    int32_t *counts, *ei, *ti, *rop;
    moe_bf16_t *rows, *rows_g, *fin_out;
    uint8_t *codes, *mx_codes, *mx_scales;
    float *qscale;
    HIP_OK(hipMalloc((void **)&counts, (size_t)(E + 1) * sizeof(int32_t)));
    HIP_OK(hipMalloc((void **)&ei, a * sizeof(int32_t)));
    HIP_OK(hipMalloc((void **)&ti, a * sizeof(int32_t)));
    HIP_OK(hipMalloc((void **)&rop, a * sizeof(int32_t)));
    /* rows >= counts[E] stay unwritten: start them at zero for a defined read-back */
    HIP_OK(hipMalloc((void **)&rows, a * row_b));
    HIP_OK(hipMalloc((void **)&rows_g, a * row_b));
    HIP_OK(hipMalloc((void **)&codes, a * (size_t)D));
    HIP_OK(hipMalloc((void **)&qscale, a * sizeof(float)));
    HIP_OK(hipMalloc((void **)&fin_out, (size_t)T * row_b));
    HIP_OK(hipMalloc((void **)&mx_codes, (size_t)T * D));
    HIP_OK(hipMalloc((void **)&mx_scales, (size_t)T * (D / 32) + 1));
    HIP_OK(hipMemset(rows, 0, a * row_b));
    HIP_OK(hipMemset(rows_g, 0, a * row_b));
    HIP_OK(hipMemset(codes, 0, a * (size_t)D));
    HIP_OK(hipMemset(qscale, 0, a * sizeof(float)));
    HIP_OK(hipMemset(mx_codes, 0, (size_t)T * D));
    HIP_OK(hipMemset(mx_scales, 0, (size_t)T * (D / 32) + 1));
    const size_t ws_bytes = moe_shuffle_workspace_bytes(T, E, K);
    const size_t gws_bytes = moe_gather_scale_workspace_bytes(T, (int32_t)a);
    const size_t sws_bytes = moe_scatter_add_workspace_bytes(T, (int32_t)a);
    void *ws = NULL, *gws = NULL, *sws = NULL;
    HIP_OK(hipMalloc(&ws, ws_bytes ? ws_bytes : 1));
    HIP_OK(hipMalloc(&gws, gws_bytes ? gws_bytes : 1));
    HIP_OK(hipMalloc(&sws, sws_bytes ? sws_bytes : 1));

    /* scores are (T, E) row-major: element strides E and 1 */
    MOE_OK(moe_shuffle(scores, E, 1, T, E, K, NULL, counts, ei, ti, rop, ws, ws_bytes, stream));
    /* counts[E] (on the device) bounds the valid rows of every later call */
    const int32_t *valid = counts + E;
    MOE_OK(moe_gather_scale(x, T, D, ti, ei, (int32_t)a, scores, E, 1, E, valid, rows_g, gws,
                            gws_bytes, stream));
    MOE_OK(moe_gather_scale_by_token(x, T, D, rop, K, ei, (int32_t)a, scores, E, 1, E, valid,
                                     rows, stream));
    MOE_OK(moe_gather_scale_quant(x, T, D, ti, ei, (int32_t)a, scores, E, 1, E, NULL, valid,
                                  codes, qscale, stream));
    MOE_OK(moe_scatter_add(out_g, T, y, ti, (int32_t)a, D, valid, sws, sws_bytes, stream));
    MOE_OK(moe_scatter_add_by_token(out, T, y, rop, K, (int32_t)a, D, valid, stream));
    MOE_OK(moe_finalize_rmsnorm(y, (int64_t)a, w, rop, shared, gamma, eps, T, K, D, 0, fin_out,
                                mx ? mx_codes : NULL, mx ? mx_scales : NULL, stream));
    HIP_OK(hipStreamSynchronize(stream));

    FILE *fout = fopen(argv[2], "wb");
    if (!fout) {
        perror(argv[2]);
        return 1;
    }
    write_back(fout, counts, (size_t)(E + 1) * sizeof(int32_t));
    write_back(fout, ei, a * sizeof(int32_t));
    write_back(fout, ti, a * sizeof(int32_t));
    write_back(fout, rop, a * sizeof(int32_t));
    write_back(fout, rows, a * row_b);
    write_back(fout, rows_g, a * row_b);
    write_back(fout, codes, a * (size_t)D);
    write_back(fout, qscale, a * sizeof(float));
    write_back(fout, out, (size_t)T * row_b);
    write_back(fout, out_g, (size_t)T * row_b);
    write_back(fout, fin_out, (size_t)T * row_b);
    write_back(fout, mx_codes, (size_t)T * D);
    write_back(fout, mx_scales, (size_t)T * (D / 32));
    fclose(fout);

    void *dev_bufs[] = {sws, gws, ws, mx_scales, mx_codes, fin_out, qscale, codes, rows_g,
                        rows, rop, ti, ei, counts, gamma, shared, w, out_g, out, y, x, scores};
    for (size_t i = 0; i < sizeof dev_bufs / sizeof dev_bufs[0]; ++i) HIP_OK(hipFree(dev_bufs[i]));
    HIP_OK(hipStreamDestroy(stream));
    void *host_bufs[] = {h_scores, h_x, h_y, h_out, h_w, h_shared, h_gamma};
    for (size_t i = 0; i < sizeof host_bufs / sizeof host_bufs[0]; ++i) free(host_bufs[i]);
    printf("done\n");
    return 0;
}
