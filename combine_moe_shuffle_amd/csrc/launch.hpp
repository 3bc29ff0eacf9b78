// Internal launchers, one per kernel family. Arguments are validated by the C
// ABI layer (api.hip) before any of these is called; each returns the HIP
// status of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// shuffle.hip
size_t shuffle_workspace_bytes(int T, int E, int K);
hipError_t launch_shuffle(const float* scores, int64_t st, int64_t se, int T, int E,
                          int K, const int* vtc, int* counts, int* expert_indices,
                          int* token_indices, int* row_of_pair, void* workspace,
                          hipStream_t stream);

// gather.hip
// The rows of each token in token_indices' valid rows [0, V), as a CSR in a
// workspace of scatter_add_workspace_bytes(T, a): start[0..T], list[0..V)
// (the order inside a token's list is not fixed). Tokens outside [0, T) are
// left out.
hipError_t launch_token_lists(const int* ti, int T, int a, const int* valid_rows,
                              void* workspace, const int** start, const int** list,
                              hipStream_t stream);
hipError_t launch_gather_scale(const uint16_t* x, int T, int D, const int* ti,
                               const int* ei, int a, const float* scores, int64_t st,
                               int64_t se, int E, const int* valid_rows, uint16_t* out,
                               void* workspace, hipStream_t stream);
hipError_t launch_gather_scale_by_token(const uint16_t* x, int T, int D,
                                        const int* row_of_pair, int K, const int* ei,
                                        int a, const float* scores, int64_t st,
                                        int64_t se, int E, const int* valid_rows,
                                        uint16_t* out, hipStream_t stream);
hipError_t launch_gather_scale_quant(const uint16_t* x, int T, int D, const int* ti,
                                     const int* ei, int a, const float* scores,
                                     int64_t st, int64_t se, int E, const float* scale_ub,
                                     const int* valid_rows, uint8_t* out_fp8,
                                     float* out_scale, hipStream_t stream);

// combine.hip
size_t scatter_add_workspace_bytes(int T, int a);
hipError_t launch_scatter_add(uint16_t* out, int T, const uint16_t* in, const int* ti,
                              int a, int D, const int* valid_rows, void* workspace,
                              hipStream_t stream);
size_t scatter_add_padded_workspace_bytes(int T, int T_K, int E);
hipError_t launch_scatter_add_padded(const uint16_t* in, int EP, int T_K, const int* counts,
                                     int E, const int* ti, uint16_t* out, int T, int D,
                                     void* workspace, hipStream_t stream);
hipError_t launch_scatter_add_padded_by_token(const uint16_t* in, int EP, int T_K,
                                              const int* counts, int E, const int* row_of_pair,
                                              int K, uint16_t* out, int T, int D,
                                              hipStream_t stream);
hipError_t launch_scatter_add_by_token(uint16_t* out, int T, const uint16_t* in,
                                       const int* row_of_pair, int K, int a, int D,
                                       const int* valid_rows, hipStream_t stream);

// reorder.hip: expert-parallel re-sort and its inverse
constexpr int kMaxShufflingSegments = 4096;  // (c_hi - c_lo) * EP
constexpr int kMaxShufflingRanks = 64;
size_t shuffling_workspace_bytes(int nseg, int64_t em_rows);
hipError_t launch_shuffling(bool inverse, const uint16_t* in, int64_t in_rows, uint16_t* out,
                            int64_t out_rows, int D, const int* counts, int EP, int C, int c_lo,
                            int c_hi, int64_t rank_stride, int* out_counts, void* workspace,
                            hipStream_t stream);

// finalize.hip
hipError_t launch_finalize_rmsnorm(const uint16_t* y, int64_t rows, const void* w,
                                   const int* row_of_pair, const uint16_t* shared,
                                   const uint16_t* gamma, float eps, int T, int K, int D,
                                   uint32_t flags, uint16_t* out, uint8_t* mx_codes,
                                   uint8_t* mx_scales, hipStream_t stream);
hipError_t launch_finalize_mhc(const uint16_t* y, int64_t rows, const void* w,
                               const int* row_of_pair, const uint16_t* shared,
                               const uint16_t* residual, const float* post, const float* comb,
                               const float* pre, const uint16_t* gamma, float eps, int T, int K,
                               int D, int hc, uint32_t flags, uint16_t* residual_out,
                               uint16_t* out, uint8_t* mx_codes, uint8_t* mx_scales,
                               hipStream_t stream);
hipError_t launch_convert_check(const float* in, int64_t n, uint16_t* bf16_out,
                                uint8_t* e4m3_out, hipStream_t stream);

// floor.hip: latency floors of the finalize's launch shape
int launch_floor_threads(int T, int D);
hipError_t launch_floor(int kind, int T, int D, const void* src, void* dst,
                        hipStream_t stream);

// Row-slice layout of the streaming kernels: a row of D bf16 values is
// nch = D/8 chunks of 16 bytes; a wave covers one slice of 64*cpl chunks,
// lane l taking chunks base + j*64 + l (j < cpl), so every load and store
// instruction of the wave touches 1 KiB of contiguous memory.
struct SliceShape {
  int cpl;  // chunks per lane
  int nsl;  // slices per row
};
// The entry of `allowed` whose slice count is <= max_slices and that wastes
// the fewest lanes; among equals, the earlier entry.
SliceShape pick_slices(int nch, const int* allowed, int n_allowed, int max_slices);

// Instantiate LAUNCH(cpl) for the run-time chunks-per-lane value (1..8).
#define MOE_DISPATCH_CPL(CPLV, LAUNCH) \
  switch (CPLV) {                      \
    case 1: LAUNCH(1); break;          \
    case 2: LAUNCH(2); break;          \
    case 3: LAUNCH(3); break;          \
    case 4: LAUNCH(4); break;          \
    case 5: LAUNCH(5); break;          \
    case 6: LAUNCH(6); break;          \
    case 7: LAUNCH(7); break;          \
    default: LAUNCH(8); break;         \
  }

}  // namespace moe
