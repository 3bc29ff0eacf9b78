/*
 * A plain C consumer of libmoe_shuffle.so: it uses nothing but
 * include/moe_shuffle.h and the HIP runtime API, no Python and no torch.
 *
 *     c_abi_consumer IN OUT
 *
 * IN holds int32 T, E, K, D, then scores (T*E fp32), x (T*D bf16), y (T*K*D
 * bf16) and out0 (T*D bf16). The program runs moe_shuffle ->
 * moe_gather_scale_by_token -> moe_scatter_add_by_token (out starts as out0)
 * on the GPU and writes OUT: counts (E+1 int32), expert_indices,
 * token_indices (T*K int32 each), row_of_pair (T*K int32), rows (T*K*D
 * bf16) and out (T*D bf16). Every status is checked; on an error it prints
 * the library's message and exits with status 1.
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
    void *h_scores = read_exact(fin, (size_t)T * E * sizeof(float));
    void *h_x = read_exact(fin, (size_t)T * D * 2);
    void *h_y = read_exact(fin, a * D * 2);
    void *h_out = read_exact(fin, (size_t)T * D * 2);
    fclose(fin);

    printf("moe_shuffle ABI %d: T=%d E=%d K=%d D=%d\n", moe_abi_version(), T, E, K, D);
    fflush(stdout);

    hipStream_t stream;
    HIP_OK(hipStreamCreate(&stream));
    float *scores = (float *)to_device(h_scores, (size_t)T * E * sizeof(float));
    moe_bf16_t *x = (moe_bf16_t *)to_device(h_x, (size_t)T * D * 2);
    moe_bf16_t *y = (moe_bf16_t *)to_device(h_y, a * D * 2);
    moe_bf16_t *out = (moe_bf16_t *)to_device(h_out, (size_t)T * D * 2);
    int32_t *counts, *ei, *ti, *rop;
    moe_bf16_t *rows;
    HIP_OK(hipMalloc((void **)&counts, (size_t)(E + 1) * sizeof(int32_t)));
    HIP_OK(hipMalloc((void **)&ei, a * sizeof(int32_t)));
    HIP_OK(hipMalloc((void **)&ti, a * sizeof(int32_t)));
    HIP_OK(hipMalloc((void **)&rop, a * sizeof(int32_t)));
    HIP_OK(hipMalloc((void **)&rows, a * D * 2));  /* rows >= counts[E] stay unwritten */
    const size_t ws_bytes = moe_shuffle_workspace_bytes(T, E, K);
    void *ws = NULL;
    HIP_OK(hipMalloc(&ws, ws_bytes ? ws_bytes : 1));

    /* scores are (T, E) row-major: element strides E and 1 */
    MOE_OK(moe_shuffle(scores, E, 1, T, E, K, NULL, counts, ei, ti, rop, ws, ws_bytes, stream));
    /* counts[E] (on the device) bounds the valid rows of both later calls */
    MOE_OK(moe_gather_scale_by_token(x, T, D, rop, K, ei, (int32_t)a, scores, E, 1, E,
                                     counts + E, rows, stream));
    MOE_OK(moe_scatter_add_by_token(out, T, y, rop, K, (int32_t)a, D, counts + E, stream));
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
    write_back(fout, rows, a * D * 2);
    write_back(fout, out, (size_t)T * D * 2);
    fclose(fout);

    HIP_OK(hipFree(ws));
    HIP_OK(hipFree(rows));
    HIP_OK(hipFree(rop));
    HIP_OK(hipFree(ti));
    HIP_OK(hipFree(ei));
    HIP_OK(hipFree(counts));
    HIP_OK(hipFree(out));
    HIP_OK(hipFree(y));
    HIP_OK(hipFree(x));
    HIP_OK(hipFree(scores));
    HIP_OK(hipStreamDestroy(stream));
    free(h_scores);
    free(h_x);
    free(h_y);
    free(h_out);
    printf("done\n");
    return 0;
}
