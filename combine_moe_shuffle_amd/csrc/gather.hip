// Dispatch: gather token rows into expert order, times the router score,
// stored as bf16 or as FP8 E4M3 with one scale per row.
//
// [GS] "mslk/moe/gather_scatter.py": gather_scale_dense_tokens,
// gather_scale_quant_dense_tokens and their kernels.
//
// The kernels stream rows in the slice layout of launch.hpp: each wave owns
// 64*cpl 16-byte chunks of one row, one 1 KiB contiguous access per
// instruction. Per-row indices and the score are wave-uniform scalar loads.
//
//  gather_rows    one (output row, slice) per wave, output-row order.
//  gather_tokens  one (token, slice) per wave: the token's slice is loaded
//                 once and written to each of its K rows through the inverse
//                 map, so x is read from memory once however large K is.
//  gather_lists   the same from token_indices, through per-token row lists
//                 built first; gather_scan, for up to 1024 rows, has each
//                 wave find its token's rows itself instead.
//  quant_rows     one output row per workgroup (its slices spread over the
//                 waves); the row stays in registers between the row-max
//                 reduction (wave max + LDS across waves) and the quantising
//                 pass, so x is read once (the pages re-read it from L2).
#include "device.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kRowWaves = 4;  // waves per workgroup for the per-slice kernels

__device__ __forceinline__ int clamp_count(const int* p, int hi) {
  if (!p) return hi;
  int v = *p;
  return v < 0 ? 0 : (v > hi ? hi : v);
}

// out[dst chunk] = bf16(f32(src chunk) * s) over this lane's chunks of a
// slice. FULL: the whole slice is inside the row, so no lane needs a bounds
// test and the loads, conversions and stores are straight-line code (a
// per-chunk branch splits them into blocks that reuse the store-data
// registers, which makes every store wait for the previous one).
template <int CPL, bool FULL>
__device__ __forceinline__ void scale_slice(const uint16_t* __restrict__ src,
                                            uint16_t* __restrict__ dst, float s, int base,
                                            int nch) {
  u32x4 v[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = base + j * kWave;
    if (FULL || c < nch) v[j] = ld16(src + c * kChunk);
  }
  u32x4 o[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    float f[8];
    unpack8(v[j], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = f[i] * s;
    o[j] = pack8(f);
  }
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = base + j * kWave;
    if (FULL || c < nch) st16_stream(dst + c * kChunk, o[j]);
  }
}

template <int CPL>
__global__ __launch_bounds__(kRowWaves* kWave) void gather_rows_kernel(
    const uint16_t* __restrict__ x, int T, int E, int D, const int* __restrict__ ti,
    const int* __restrict__ ei, int a, const float* __restrict__ scores, int64_t st,
    int64_t se, const int* __restrict__ vrows, uint16_t* __restrict__ out, int nsl) {
  const int lane = lane_id();
  const int64_t unit =
      static_cast<int64_t>(blockIdx.x) * kRowWaves + uniform(threadIdx.x >> 6);
  const int row = static_cast<int>(unit / nsl);
  const int sl = static_cast<int>(unit - static_cast<int64_t>(row) * nsl);
  if (row >= a) return;
  const int V = clamp_count(vrows, a);
  if (row >= V) return;
  const int t = ti[row];
  const int e = ei[row];
  if (static_cast<unsigned>(t) >= static_cast<unsigned>(T) ||
      static_cast<unsigned>(e) >= static_cast<unsigned>(E))
    return;  // out-of-range index: row skipped
  const float s = scores[static_cast<int64_t>(t) * st + static_cast<int64_t>(e) * se];
  const int nch = D >> 3;
  const uint16_t* src = x + static_cast<int64_t>(t) * D;
  uint16_t* dst = out + static_cast<int64_t>(row) * D;
  const int slice0 = sl * kWave * CPL;
  if (slice0 + kWave * CPL <= nch)
    scale_slice<CPL, true>(src, dst, s, slice0 + lane, nch);
  else
    scale_slice<CPL, false>(src, dst, s, slice0 + lane, nch);
}

// One token's slice, written to each of its valid rows scaled by that row's
// score. Lane k holds slot k's row (my_r) and score (my_s); `valid` marks the
// slots to write.
template <int CPL, bool FULL>
__device__ __forceinline__ void scatter_token_slice(const u32x4 (&v)[CPL],
                                                    uint16_t* __restrict__ out, int D, int my_r,
                                                    float my_s, uint64_t valid, int base,
                                                    int nch) {
  for (uint64_t m = valid; m; m &= m - 1) {
    const int k = __builtin_ctzll(m);
    const int r = __builtin_amdgcn_readlane(my_r, k);
    const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), k));
    uint16_t* dst = out + static_cast<int64_t>(r) * D;
    u32x4 o[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      float f[8];
      unpack8(v[j], f);
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = f[i] * s;
      o[j] = pack8(f);
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = base + j * kWave;
      if (FULL || c < nch) st16_stream(dst + c * kChunk, o[j]);
    }
  }
}

// Dependent loads per wave: the token's slot rows; then, at once, the x slice
// and every slot's expert id (lane k fetches slot k's); then every slot's
// score; then the K row writes.
template <int CPL, bool FULL>
__device__ __forceinline__ void gather_token(const uint16_t* __restrict__ src,
                                             uint16_t* __restrict__ out, int D,
                                             const float* __restrict__ srow, int64_t se,
                                             const int* __restrict__ ei, int E, int my_r,
                                             uint64_t valid, int base, int nch) {
  // plain loads for x: measured faster here than non-temporal ones
  u32x4 v[CPL];
  const int my_e = my_r >= 0 ? ei[my_r] : -1;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = base + j * kWave;
    if (FULL || c < nch) v[j] = ld16(src + c * kChunk);
  }
  const bool ok = static_cast<unsigned>(my_e) < static_cast<unsigned>(E);  // else skipped
  const float my_s = ok ? srow[static_cast<int64_t>(my_e) * se] : 0.0f;
  scatter_token_slice<CPL, FULL>(v, out, D, my_r, my_s, valid & __ballot(ok), base, nch);
}

template <int CPL>
__global__ __launch_bounds__(kRowWaves* kWave) void gather_tokens_kernel(
    const uint16_t* __restrict__ x, int T, int E, int D, const int* __restrict__ rop, int K,
    const int* __restrict__ ei, int a, const float* __restrict__ scores, int64_t st,
    int64_t se, const int* __restrict__ vrows, uint16_t* __restrict__ out, int nsl) {
  const int lane = lane_id();
  const int64_t unit =
      static_cast<int64_t>(blockIdx.x) * kRowWaves + uniform(threadIdx.x >> 6);
  const int t = static_cast<int>(unit / nsl);
  const int sl = static_cast<int>(unit - static_cast<int64_t>(t) * nsl);
  if (t >= T) return;
  const int V = clamp_count(vrows, a);
  const int* rp = rop + static_cast<int64_t>(t) * K;
  // lane k holds slot k's row (K <= 64); invalid slots become -1
  int my_r = lane < K ? rp[lane] : -1;
  if (my_r >= V) my_r = -1;
  const uint64_t valid = __ballot(my_r >= 0);
  if (valid == 0) return;
  const int nch = D >> 3;
  const uint16_t* src = x + static_cast<int64_t>(t) * D;
  const float* srow = scores + static_cast<int64_t>(t) * st;
  const int slice0 = sl * kWave * CPL;
  if (slice0 + kWave * CPL <= nch)
    gather_token<CPL, true>(src, out, D, srow, se, ei, E, my_r, valid, slice0 + lane, nch);
  else
    gather_token<CPL, false>(src, out, D, srow, se, ei, E, my_r, valid, slice0 + lane, nch);
}

// The same as gather_tokens_kernel with each token's rows taken from a CSR
// of token_indices (launch_token_lists) instead of row_of_pair: up to 64 rows
// per pass, in any order (rows are written, not accumulated).
template <int CPL>
__global__ __launch_bounds__(kRowWaves* kWave) void gather_lists_kernel(
    const uint16_t* __restrict__ x, int T, int E, int D, const int* __restrict__ start,
    const int* __restrict__ list, const int* __restrict__ ei, const float* __restrict__ scores,
    int64_t st, int64_t se, uint16_t* __restrict__ out, int nsl) {
  const int lane = lane_id();
  const int64_t unit =
      static_cast<int64_t>(blockIdx.x) * kRowWaves + uniform(threadIdx.x >> 6);
  const int t = static_cast<int>(unit / nsl);
  const int sl = static_cast<int>(unit - static_cast<int64_t>(t) * nsl);
  if (t >= T) return;
  const int beg = start[t];
  const int n = start[t + 1] - beg;
  const int nch = D >> 3;
  const uint16_t* src = x + static_cast<int64_t>(t) * D;
  const float* srow = scores + static_cast<int64_t>(t) * st;
  const int slice0 = sl * kWave * CPL;
  const bool full = slice0 + kWave * CPL <= nch;
  for (int c0 = 0; c0 < n; c0 += kWave) {
    const int my_r = lane < n - c0 ? list[beg + c0 + lane] : -1;
    const uint64_t valid = __ballot(my_r >= 0);
    if (full)
      gather_token<CPL, true>(src, out, D, srow, se, ei, E, my_r, valid, slice0 + lane, nch);
    else
      gather_token<CPL, false>(src, out, D, srow, se, ei, E, my_r, valid, slice0 + lane, nch);
  }
}

// Small general gathers (up to kScanRows rows): each (token, slice) wave
// finds its token's rows itself (for_token_rows), with no row-list build and
// so no launch before it, and writes them up to 64 at a time as
// gather_lists_kernel does.
constexpr int kScanRows = 1024;
constexpr int kScanChunks = kScanRows / kWave;
template <int CPL>
__global__ __launch_bounds__(kRowWaves* kWave) void gather_scan_kernel(
    const uint16_t* __restrict__ x, int T, int E, int D, const int* __restrict__ ti,
    const int* __restrict__ ei, int a, const float* __restrict__ scores, int64_t st,
    int64_t se, const int* __restrict__ vrows, uint16_t* __restrict__ out, int nsl) {
  __shared__ int stage[kRowWaves][kWave];
  const int lane = lane_id();
  const int wv = uniform(threadIdx.x >> 6);
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * kRowWaves + wv;
  const int t = static_cast<int>(unit / nsl);
  const int sl = static_cast<int>(unit - static_cast<int64_t>(t) * nsl);
  if (t >= T) return;
  const int V = clamp_count(vrows, a);
  int tv[kScanChunks];
#pragma unroll
  for (int c = 0; c < kScanChunks; ++c) {
    const int r = c * kWave + lane;
    tv[c] = r < V ? ti[r] : -1;
  }
  const int nch = D >> 3;
  const uint16_t* src = x + static_cast<int64_t>(t) * D;
  const float* srow = scores + static_cast<int64_t>(t) * st;
  const int slice0 = sl * kWave * CPL;
  const bool full = slice0 + kWave * CPL <= nch;
  for_token_rows(tv, V, t, lane, stage[wv], [&](int rows, int nb) {
    const int my_r = lane < nb ? rows : -1;
    const uint64_t valid = __ballot(my_r >= 0);
    if (full)
      gather_token<CPL, true>(src, out, D, srow, se, ei, E, my_r, valid, slice0 + lane, nch);
    else
      gather_token<CPL, false>(src, out, D, srow, se, ei, E, my_r, valid, slice0 + lane, nch);
  });
}

constexpr float kRowwiseEps = 1e-12f;

template <int CPL>
__global__ __launch_bounds__(1024) void quant_rows_kernel(
    const uint16_t* __restrict__ x, int T, int E, int D, const int* __restrict__ ti,
    const int* __restrict__ ei, int a, const float* __restrict__ scores, int64_t st,
    int64_t se, const float* __restrict__ scale_ub, const int* __restrict__ vrows,
    uint8_t* __restrict__ out, float* __restrict__ out_scale) {
  __shared__ float wave_max_lds[16];
  const int row = blockIdx.x;
  const int V = clamp_count(vrows, a);
  if (row >= V) return;
  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int t = ti[row];
  const int e = ei[row];
  if (static_cast<unsigned>(t) >= static_cast<unsigned>(T) ||
      static_cast<unsigned>(e) >= static_cast<unsigned>(E))
    return;  // out-of-range index: row skipped (uniform over the workgroup)
  const float s = scores[static_cast<int64_t>(t) * st + static_cast<int64_t>(e) * se];
  const int nch = D >> 3;
  const uint16_t* src = x + static_cast<int64_t>(t) * D;
  const int base = wave * kWave * CPL + lane;

  u32x4 v[CPL];
  if (wave * kWave * CPL + kWave * CPL <= nch) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) v[j] = ld16(src + (base + j * kWave) * kChunk);
  } else {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = base + j * kWave;
      v[j] = c < nch ? ld16(src + c * kChunk) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  float m = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    float f[8];
    unpack8(v[j], f);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = __builtin_fmaxf(m, __builtin_fabsf(f[i] * s));
  }
  m = wave_max(m);
  if (lane == 0) wave_max_lds[wave] = m;
  __syncthreads();
  m = wave_max_lds[0];
  for (int w = 1; w < nwaves; ++w) m = __builtin_fmaxf(m, wave_max_lds[w]);
  // clamp the row max, then the quantisation multiplier and its reciprocal
  if (scale_ub) m = __builtin_fminf(__builtin_fmaxf(m, kRowwiseEps), *scale_ub);
  else m = __builtin_fmaxf(m, kRowwiseEps);
  const float mult = kE4M3Max / m;
  if (threadIdx.x == 0) out_scale[row] = 1.0f / mult;

  uint8_t* dst = out + static_cast<int64_t>(row) * D;
  u32x2 w[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    float f[8];
    unpack8(v[j], f);
    float q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = clamp448((f[i] * s) * mult);
    w[j].x = pack_e4m3x4(q[0], q[1], q[2], q[3]);
    w[j].y = pack_e4m3x4(q[4], q[5], q[6], q[7]);
  }
  if (wave * kWave * CPL + kWave * CPL <= nch) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) st8_stream(dst + (base + j * kWave) * kChunk, w[j]);
  } else {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = base + j * kWave;
      if (c < nch) st8_stream(dst + c * kChunk, w[j]);
    }
  }
}

// Per-slice shape of the independent-slice kernels: the least lane waste,
// and among equals the fewest chunks per lane (more, shorter waves measured
// slightly faster on the 7168-wide rows).
SliceShape stream_shape(int nch) {
  static const int allowed[] = {1, 2, 3, 4, 5, 6, 7, 8};
  return pick_slices(nch, allowed, 8, 1 << 20);
}

}  // namespace

SliceShape pick_slices(int nch, const int* allowed, int n_allowed, int max_slices) {
  // least wasted lanes first; among equals, the earlier entry of `allowed`
  SliceShape best{allowed[n_allowed - 1], (nch + kWave * allowed[n_allowed - 1] - 1) /
                                              (kWave * allowed[n_allowed - 1])};
  long best_waste = -1;
  for (int i = 0; i < n_allowed; ++i) {
    const int cpl = allowed[i];
    const int per = kWave * cpl;
    const int nsl = (nch + per - 1) / per;
    if (nsl > max_slices) continue;
    const long waste = static_cast<long>(nsl) * per - nch;
    if (best_waste < 0 || waste < best_waste) {
      best_waste = waste;
      best = SliceShape{cpl, nsl};
    }
  }
  return best;
}

hipError_t launch_gather_scale(const uint16_t* x, int T, int D, const int* ti,
                               const int* ei, int a, const float* scores, int64_t st,
                               int64_t se, int E, const int* valid_rows, uint16_t* out,
                               void* workspace, hipStream_t stream) {
  const SliceShape sh = stream_shape(D / kChunk);
  if (workspace) {
    // token order: each x row read once, written to its rows through a CSR
    // of token_indices built in the workspace, or for small inputs found by
    // each wave itself
    const int64_t tunits = static_cast<int64_t>(T) * sh.nsl;
    const dim3 tgrid(static_cast<unsigned>((tunits + kRowWaves - 1) / kRowWaves));
    if (a <= kScanRows) {
#define LS(C)                                                                              \
  hipLaunchKernelGGL(gather_scan_kernel<C>, tgrid, dim3(kRowWaves * kWave), 0, stream, x, T, \
                     E, D, ti, ei, a, scores, st, se, valid_rows, out, sh.nsl)
      MOE_DISPATCH_CPL(sh.cpl, LS)
#undef LS
      return hipGetLastError();
    }
    const int* start;
    const int* list;
    const hipError_t e = launch_token_lists(ti, T, a, valid_rows, workspace, &start, &list,
                                            stream);
    if (e != hipSuccess) return e;
#define LT(C)                                                                              \
  hipLaunchKernelGGL(gather_lists_kernel<C>, tgrid, dim3(kRowWaves * kWave), 0, stream, x, T, \
                     E, D, start, list, ei, scores, st, se, out, sh.nsl)
    MOE_DISPATCH_CPL(sh.cpl, LT)
#undef LT
    return hipGetLastError();
  }
  // row order: one wave per (row, slice), x re-read once per route
  const int64_t units = static_cast<int64_t>(a) * sh.nsl;
  const dim3 grid(static_cast<unsigned>((units + kRowWaves - 1) / kRowWaves));
  const dim3 block(kRowWaves * kWave);
#define L(C)                                                                             \
  hipLaunchKernelGGL(gather_rows_kernel<C>, grid, block, 0, stream, x, T, E, D, ti, ei, a, scores, \
                     st, se, valid_rows, out, sh.nsl)
  MOE_DISPATCH_CPL(sh.cpl, L)
#undef L
  return hipGetLastError();
}

hipError_t launch_gather_scale_by_token(const uint16_t* x, int T, int D,
                                        const int* row_of_pair, int K, const int* ei,
                                        int a, const float* scores, int64_t st,
                                        int64_t se, int E, const int* valid_rows,
                                        uint16_t* out, hipStream_t stream) {
  const SliceShape sh = stream_shape(D / kChunk);
  const int64_t units = static_cast<int64_t>(T) * sh.nsl;
  const dim3 grid(static_cast<unsigned>((units + kRowWaves - 1) / kRowWaves));
  const dim3 block(kRowWaves * kWave);
#define L(C)                                                                                 \
  hipLaunchKernelGGL(gather_tokens_kernel<C>, grid, block, 0, stream, x, T, E, D, row_of_pair, K, \
                     ei, a, scores, st, se, valid_rows, out, sh.nsl)
  MOE_DISPATCH_CPL(sh.cpl, L)
#undef L
  return hipGetLastError();
}

hipError_t launch_gather_scale_quant(const uint16_t* x, int T, int D, const int* ti,
                                     const int* ei, int a, const float* scores,
                                     int64_t st, int64_t se, int E, const float* scale_ub,
                                     const int* valid_rows, uint8_t* out_fp8,
                                     float* out_scale, hipStream_t stream) {
  // one row per workgroup of up to 16 waves; among the shapes that waste the
  // fewest lanes, the fewest waves (more chunks per lane): a 5120-wide row in
  // one wave of 10 chunks per lane measured 15 % faster than in five waves of
  // 2, with fewer rows sharing a workgroup barrier. 10 chunks per lane take
  // 121 registers; more would spill under the 1024-thread launch bound.
  static const int allowed[] = {10, 8, 7, 6, 5, 4, 3, 2, 1};
  const SliceShape sh = pick_slices(D / kChunk, allowed, 9, 16);
  const dim3 grid(static_cast<unsigned>(a));
  const dim3 block(sh.nsl * kWave);
#define L(C)                                                                             \
  hipLaunchKernelGGL(quant_rows_kernel<C>, grid, block, 0, stream, x, T, E, D, ti, ei, a, scores, \
                     st, se, scale_ub, valid_rows, out_fp8, out_scale)
  if (sh.cpl == 10) {
    L(10);
  } else {
    MOE_DISPATCH_CPL(sh.cpl, L)
  }
#undef L
  return hipGetLastError();
}

}  // namespace moe
