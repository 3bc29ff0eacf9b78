// The MoE tail on one GPU: weighted top-k reduction of the permuted expert
// outputs, shared-expert add, RMSNorm, and optionally MXFP8 (E4M3 codes with a
// UE8M0 power-of-two scale per 32 elements) of the normalised row.
//
// [K3] "vllm ... kimi_k3 ... allreduce_rmsnorm_reduce_scatter_early_exit",
// routed role: top-k finalize (fp32 sum of weight * row over the slots whose
// permuted row is >= 0) and RMSNorm (row sum of squares, rsqrt(sum/D + eps),
// bf16(x * inv * gamma)); its default mode rounds each square to bf16.
// [MH] "vllm ... deepseek_v41 ... all_reduce_mhc": AllReduceMHC.finalize (fp32
// weights, the shared-expert output folded into the same pass) and
// _LamportMHCDeviceKernel (fp32 squares; MXFP8 of the bf16 output from the
// block max times 1/448, rounded to a power-of-two scale).
//
// The pages spread one token over a thread-block cluster and reduce through
// distributed shared memory; gfx950 has no clusters, so one workgroup of up to
// 16 waves owns a token: each wave holds a slice of the row in registers, the
// sum of squares goes wave-wide by shuffles and across waves through LDS, and
// the row is written once. All K expert rows of a chunk are loaded before the
// first multiply-add (the pages' prefetch of every top-k row at once).
// The MXFP8 block of 32 elements is 4 adjacent chunks = 4 adjacent lanes, so
// its max is two lane swaps.
#include "device.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kMaxWaves = 16;

// UE8M0 exponent byte of a block max: ceil(log2(amax * fp32(1/448))) + 127,
// clamped to [0, 254]; 0 for a zero block. The ceiling comes from the bits of
// p: a normal p = 2^(ef-127) * 1.m is an exact power iff m == 0; a subnormal
// p = m * 2^-149 has ceil(log2 p) = ceil(log2 m) - 149.
__device__ __forceinline__ uint32_t ue8m0_of(float amax) {
  const float p = amax * (1.0f / kE4M3Max);
  const uint32_t bits = __float_as_uint(p);
  const int ef = static_cast<int>((bits >> 23) & 0xFFu);
  const uint32_t m = bits & 0x7FFFFFu;
  int c;
  if (ef == 0) {
    if (m == 0) return 0u;
    c = (32 - __clz(static_cast<int>(m - 1u))) - 149;  // m == 1 -> -149
  } else {
    c = ef - 127 + (m != 0u ? 1 : 0);
  }
  int byte = c + 127;
  byte = byte < 0 ? 0 : (byte > 254 ? 254 : byte);
  return static_cast<uint32_t>(byte);
}

// Loads the expert rows of slots [k0, k0+G). Every load is unconditional:
// a slot that is not held (or past K) re-reads `safe`, a held row of the same
// token (an L2 hit), so all G*CPL loads issue back to back.
template <int CPL, int G, bool FULL>
__device__ __forceinline__ void load_slots(u32x4 (&buf)[G][CPL], const uint16_t* __restrict__ y,
                                           int D, int nch, int base, int my_r, int K, int k0,
                                           int safe) {
#pragma unroll
  for (int q = 0; q < G; ++q) {
    const int k = k0 + q;
    const int r = __builtin_amdgcn_readlane(my_r, min(k, kWave - 1));
    const int rr = (k < K && r >= 0) ? r : safe;
    const uint16_t* src = y + static_cast<int64_t>(rr) * D;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = base + j * kWave;
      if (FULL || c < nch) buf[q][j] = ld16_stream(src + c * kChunk);
    }
  }
}

// acc = fma(w_k, row_k, acc) over the held slots of the group, in slot order
// (the select keeps acc unchanged for a slot that is not held).
template <int CPL, int G, bool FULL>
__device__ __forceinline__ void fma_slots(float (&acc)[CPL][8], const u32x4 (&buf)[G][CPL],
                                          int nch, int base, int my_r, float my_w, int K,
                                          int k0) {
#pragma unroll
  for (int q = 0; q < G; ++q) {
    const int k = k0 + q;
    const int kq = min(k, kWave - 1);
    const bool held = k < K && __builtin_amdgcn_readlane(my_r, kq) >= 0;
    const float wq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), kq));
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = base + j * kWave;
      if (FULL || c < nch) {
        float f[8];
        unpack8(buf[q][j], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float v = __builtin_fmaf(wq, f[i], acc[j][i]);
          acc[j][i] = held ? v : acc[j][i];
        }
      }
    }
  }
}

// Byte offset of MXFP8 scale (row m, block column k) in the swizzled layout:
// 128-row x 4-column tiles of 512 bytes, row-tile-major; inside a tile, row m
// and column k at (m % 32) * 16 + ((m % 128) / 32) * 4 + (k % 4).
__device__ __forceinline__ int64_t swizzled_scale_offset(int m, int k, int cols) {
  const int64_t tile = static_cast<int64_t>(m >> 7) * ((cols + 3) >> 2) + (k >> 2);
  return tile * 512 + (m & 31) * 16 + ((m & 127) >> 5) * 4 + (k & 3);
}

// Per-token set-up shared by both kernels: lane k holds slot k (K <= 64), its
// permuted row (or -1) and its weight (fp32, or bf16 widened exactly with
// flags bit 1). A row >= rows is out of range and treated as not held.
__device__ __forceinline__ void load_pairs(int t, int K, int64_t rows, const void* w,
                                           const int* __restrict__ rop, uint32_t flags,
                                           int lane, int& my_r, float& my_w) {
  my_r = -1;
  my_w = 0.0f;
  if (lane < K) {
    const int64_t i = static_cast<int64_t>(t) * K + lane;
    my_r = rop[i];
    my_w = (flags & 2u) ? bf16_lo(static_cast<const uint16_t*>(w)[i])
                        : static_cast<const float*>(w)[i];
    if (my_r >= rows) my_r = -1;
  }
}

// h = bf16(sum over held slots of w_k * y[r_k] (fp32 fma, slot order)
// [+ shared]) for this lane's chunks; sh holds the shared row's chunks.
template <int CPL, int G, bool FULL>
__device__ __forceinline__ void routed_sum(u32x4 (&h)[CPL], const u32x4 (&sh)[CPL],
                                           bool has_shared, const uint16_t* __restrict__ y,
                                           int D, int nch, int base, int lane, int K, int my_r,
                                           float my_w) {
  float acc[CPL][8];
#pragma unroll
  for (int j = 0; j < CPL; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = 0.0f;
  const uint64_t held = __ballot(lane < K && my_r >= 0);
  if (held != 0) {
    const int safe = __builtin_amdgcn_readlane(my_r, __builtin_ctzll(held));
    u32x4 buf[G][CPL];
    load_slots<CPL, G, FULL>(buf, y, D, nch, base, my_r, K, 0, safe);
    fma_slots<CPL, G, FULL>(acc, buf, nch, base, my_r, my_w, K, 0);
    for (int k0 = G; k0 < K; k0 += G) {
      load_slots<CPL, G, FULL>(buf, y, D, nch, base, my_r, K, k0, safe);
      fma_slots<CPL, G, FULL>(acc, buf, nch, base, my_r, my_w, K, k0);
    }
  }
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = base + j * kWave;
    if (FULL || c < nch) {
      if (has_shared) {
        float f[8];
        unpack8(sh[j], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = acc[j][i] + f[i];
      }
      h[j] = pack8(acc[j]);
    }
  }
}

// RMSNorm of the bf16 row x (this lane's chunks) and its optional MXFP8:
// squares in fp32 (flags bit 0: rounded to bf16), summed in fp64 (lane, wave
// tree, then waves in order through LDS) and rounded once to fp32. A square
// of a bf16 value has at most 16 significant bits, so the fp64 sum is exact or
// off by a few fp64 ulps; its fp32 rounding can then depend on the reduction
// order only when the exact sum lies that close to the midpoint of two fp32
// values (one fp32 ulp is 2^29 fp64 ulps). inv = correctly rounded
// 1/sqrt(ss/D + eps);
// out = bf16((x * inv) * gamma); MXFP8 of the bf16 output.
template <int CPL, bool MX, bool FULL>
__device__ __forceinline__ void norm_out(const u32x4 (&x)[CPL], const u32x4 (&gm)[CPL],
                                         double* wave_ss, int t, int D, int nch, int base,
                                         int lane, int wave, int nwaves, float eps,
                                         uint32_t flags, uint16_t* __restrict__ out,
                                         uint8_t* __restrict__ codes,
                                         uint8_t* __restrict__ scales) {
  const int cols = D >> 5;
  // the lane's squares summed as a tree (short dependent chains; in fp64 the
  // order does not matter)
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = base + j * kWave;
    if (FULL || c < nch) {
      float hf[8];
      unpack8(x[j], hf);
      double d[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float sq = hf[i] * hf[i];
        if (flags & 1u) sq = bf16_lo(pack_bf16x2(sq, 0.0f));
        d[i] = static_cast<double>(sq);
      }
      ss = ss + (((d[0] + d[1]) + (d[2] + d[3])) + ((d[4] + d[5]) + (d[6] + d[7])));
    }
  }
  ss = wave_sum_f64(ss);
  if (lane == 0) wave_ss[wave] = ss;
  __syncthreads();
  double total = 0.0;
  for (int v = 0; v < nwaves; ++v) total = total + wave_ss[v];
  const float mean = static_cast<float>(total) / static_cast<float>(D);
  const float inv = static_cast<float>(1.0 / sqrt(static_cast<double>(mean + eps)));

  uint16_t* orow = out + static_cast<int64_t>(t) * D;
  u32x4 ob[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    float hf[8], g[8], o[8];
    unpack8(x[j], hf);
    unpack8(gm[j], g);
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (hf[i] * inv) * g[i];
    ob[j] = pack8(o);
  }
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = base + j * kWave;
    if (FULL || c < nch) st16_stream(orow + c * kChunk, ob[j]);
  }
  if constexpr (MX) {
    u32x2 cw[CPL];
    uint32_t bytes[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      // the bf16-rounded output feeds the quantiser; dead chunks hold zeros
      const int c = base + j * kWave;
      float o[8];
      unpack8((FULL || c < nch) ? ob[j] : u32x4{0u, 0u, 0u, 0u}, o);
      // block max over the 4 lanes holding this 32-element block; every lane
      // joins the swaps (nch is a multiple of 4, so a block is wholly live
      // or wholly dead)
      float am = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) am = __builtin_fmaxf(am, __builtin_fabsf(o[i]));
      am = __builtin_fmaxf(am, __shfl_xor(am, 1, kWave));
      am = __builtin_fmaxf(am, __shfl_xor(am, 2, kWave));
      bytes[j] = ue8m0_of(am);
      const float mult = __builtin_amdgcn_ldexpf(1.0f, 127 - static_cast<int>(bytes[j]));
      float q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = clamp448(o[i] * mult);
      cw[j].x = pack_e4m3x4(q[0], q[1], q[2], q[3]);
      cw[j].y = pack_e4m3x4(q[4], q[5], q[6], q[7]);
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = base + j * kWave;
      if (FULL || c < nch) {
        st8_stream(codes + static_cast<int64_t>(t) * D + c * kChunk, cw[j]);
        if ((lane & 3) == 0) {
          const int64_t so = (flags & 4u) ? swizzled_scale_offset(t, c >> 2, cols)
                                          : static_cast<int64_t>(t) * cols + (c >> 2);
          scales[so] = static_cast<uint8_t>(bytes[j]);
        }
      }
    }
  }
}

// Workgroup T + i (swizzled scales only) zeroes padding row T + i's scales.
__device__ __forceinline__ void zero_pad_scales(int t, int cols, uint8_t* __restrict__ scales) {
  for (int k = threadIdx.x; k < cols; k += blockDim.x)
    scales[swizzled_scale_offset(t, k, cols)] = 0;
}

// FULL: every wave's slice lies inside the row (D == waves * 64 * CPL * 8),
// so no chunk needs a bounds test and loads/stores are straight-line code.
// G: expert rows in flight per group (>= K where possible: one group).
template <int CPL, int G, bool MX, bool FULL>
__global__ __launch_bounds__(kMaxWaves* kWave) void finalize_kernel(
    const uint16_t* __restrict__ y, int64_t rows, const void* __restrict__ w,
    const int* __restrict__ rop, const uint16_t* __restrict__ shared,
    const uint16_t* __restrict__ gamma, float eps, int T, int K, int D, uint32_t flags,
    uint16_t* __restrict__ out, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  __shared__ double wave_ss[kMaxWaves];

  const int t = blockIdx.x;
  if (t >= T) {
    if constexpr (MX) zero_pad_scales(t, D >> 5, scales);
    return;
  }
  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int nch = D >> 3;
  const int base = wave * kWave * CPL + lane;

  int my_r;
  float my_w;
  load_pairs(t, K, rows, w, rop, flags, lane, my_r, my_w);

  // shared output and gamma are independent of the slot loop: issue early
  u32x4 sh[CPL], gm[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = base + j * kWave;
    if (FULL || c < nch) {
      if (shared) sh[j] = ld16_stream(shared + static_cast<int64_t>(t) * D + c * kChunk);
      gm[j] = ld16(gamma + c * kChunk);
    }
  }

  u32x4 h[CPL];
  routed_sum<CPL, G, FULL>(h, sh, shared != nullptr, y, D, nch, base, lane, K, my_r, my_w);
  norm_out<CPL, MX, FULL>(h, gm, wave_ss, t, D, nch, base, lane, wave, nwaves, eps, flags, out,
                          codes, scales);
}

// The mHC tail ([MH] _LamportMHCDeviceKernel) after the routed sum h:
//   for each target stream j: mixed = h * post[t][j], then for each source
//   stream s in order mixed = fma(residual[t][s], comb[t][s][j], mixed);
//   residual_out[t][j] = bf16(mixed); collapse = fma(bf16 mixed, pre[t][j],
//   collapse) over j in order; prenorm = bf16(collapse) goes through the same
//   RMSNorm (+ MXFP8). NORM = false (pre == NULL): only residual_out.
// comb is [source][target]. The mixing coefficients are per token, so every
// lane of the workgroup reads the same ones (scalar loads).
template <int CPL, int G, int HC, bool MX, bool FULL, bool NORM>
__global__ __launch_bounds__(kMaxWaves* kWave) void finalize_mhc_kernel(
    const uint16_t* __restrict__ y, int64_t rows, const void* __restrict__ w,
    const int* __restrict__ rop, const uint16_t* __restrict__ shared,
    const uint16_t* __restrict__ residual, const float* __restrict__ post,
    const float* __restrict__ comb, const float* __restrict__ pre,
    const uint16_t* __restrict__ gamma, float eps, int T, int K, int D, uint32_t flags,
    uint16_t* __restrict__ residual_out, uint16_t* __restrict__ out,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  __shared__ double wave_ss[kMaxWaves];

  const int t = blockIdx.x;
  if (t >= T) {
    if constexpr (MX) zero_pad_scales(t, D >> 5, scales);
    return;
  }
  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int nch = D >> 3;
  const int base = wave * kWave * CPL + lane;

  int my_r;
  float my_w;
  load_pairs(t, K, rows, w, rop, flags, lane, my_r, my_w);

  // shared, gamma and the hc residual streams do not depend on the slots
  u32x4 sh[CPL], gm[CPL], rs[HC][CPL];
  const uint16_t* rrow = residual + static_cast<int64_t>(t) * HC * D;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = base + j * kWave;
    if (FULL || c < nch) {
      if (shared) sh[j] = ld16_stream(shared + static_cast<int64_t>(t) * D + c * kChunk);
      if constexpr (NORM) gm[j] = ld16(gamma + c * kChunk);
#pragma unroll
      for (int s = 0; s < HC; ++s)
        rs[s][j] = ld16_stream(rrow + static_cast<int64_t>(s) * D + c * kChunk);
    }
  }
  float pm[HC], cm[HC][HC], qm[HC];
#pragma unroll
  for (int a = 0; a < HC; ++a) {
    pm[a] = post[static_cast<int64_t>(t) * HC + a];
    if constexpr (NORM) qm[a] = pre[static_cast<int64_t>(t) * HC + a];
#pragma unroll
    for (int b = 0; b < HC; ++b) cm[a][b] = comb[(static_cast<int64_t>(t) * HC + a) * HC + b];
  }

  u32x4 h[CPL];
  routed_sum<CPL, G, FULL>(h, sh, shared != nullptr, y, D, nch, base, lane, K, my_r, my_w);

  uint16_t* orow = residual_out + static_cast<int64_t>(t) * HC * D;
  u32x4 pn[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = base + j * kWave;
    if (FULL || c < nch) {
      float hf[8], rf[HC][8], col[8];
      unpack8(h[j], hf);
#pragma unroll
      for (int s = 0; s < HC; ++s) unpack8(rs[s][j], rf[s]);
#pragma unroll
      for (int i = 0; i < 8; ++i) col[i] = 0.0f;
#pragma unroll
      for (int tg = 0; tg < HC; ++tg) {
        float mx[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float m = hf[i] * pm[tg];
#pragma unroll
          for (int s = 0; s < HC; ++s) m = __builtin_fmaf(rf[s][i], cm[s][tg], m);
          mx[i] = m;
        }
        const u32x4 mb = pack8(mx);
        st16_stream(orow + static_cast<int64_t>(tg) * D + c * kChunk, mb);
        if constexpr (NORM) {
          float mf[8];
          unpack8(mb, mf);
#pragma unroll
          for (int i = 0; i < 8; ++i) col[i] = __builtin_fmaf(mf[i], qm[tg], col[i]);
        }
      }
      if constexpr (NORM) pn[j] = pack8(col);
    }
  }
  if constexpr (NORM)
    norm_out<CPL, MX, FULL>(pn, gm, wave_ss, t, D, nch, base, lane, wave, nwaves, eps, flags,
                            out, codes, scales);
}

// fp32 -> bf16 and fp32 -> E4M3 (after the +-448 clamp) through the same
// device conversions the kernels use.
__global__ void convert_kernel(const float* __restrict__ in, int64_t n,
                               uint16_t* __restrict__ bf, uint8_t* __restrict__ e4) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const float v = in[i];
  if (bf) bf[i] = static_cast<uint16_t>(pack_bf16x2(v, 0.0f) & 0xFFFFu);
  if (e4) {
    const float c = clamp448(v);
    e4[i] = static_cast<uint8_t>(pack_e4m3x4(c, 0.0f, 0.0f, 0.0f) & 0xFFu);
  }
}

}  // namespace

// up to 32 tokens: two chunks per lane (a 7168-wide row in 7 waves measured
// 0.2 us faster than in 14 at 1-32 tokens: fewer waves to launch and to meet
// at the barrier); up to 2047 tokens: one chunk per lane and up to 16 waves
// per token (latency); more: two chunks per lane, fewer waves per token
SliceShape finalize_launch_shape(int T, int D) {
  const int nch = D / kChunk;
  static const int tiny_t[] = {2, 1, 4, 8};
  static const int small_t[] = {1, 2, 4, 8};
  static const int large_t[] = {2, 4, 8, 1};
  return T <= 32   ? pick_slices(nch, tiny_t, 4, kMaxWaves)
         : T < 2048 ? pick_slices(nch, small_t, 4, kMaxWaves)
                    : pick_slices(nch, large_t, 4, kMaxWaves);
}

hipError_t launch_finalize_rmsnorm(const uint16_t* y, int64_t rows, const void* w,
                                   const int* row_of_pair, const uint16_t* shared,
                                   const uint16_t* gamma, float eps, int T, int K, int D,
                                   uint32_t flags, uint16_t* out, uint8_t* mx_codes,
                                   uint8_t* mx_scales, hipStream_t stream) {
  const int nch = D / kChunk;
  const SliceShape sh = finalize_launch_shape(T, D);
  // with swizzled MXFP8 scales, one more workgroup per padding row (up to a
  // multiple of 128 rows) zeroes that row's scales
  const int pad_rows = (mx_codes && (flags & 4u)) ? (T + 127) / 128 * 128 - T : 0;
  const dim3 grid(static_cast<unsigned>(T + pad_rows));
  const dim3 block(sh.nsl * kWave);
  const bool mx = mx_codes != nullptr;
  const bool full = sh.nsl * kWave * sh.cpl == nch;
  // rows in flight per group: the next power of two >= K (at most 8), with
  // G * cpl <= 16 to bound the registers
  const int gk = K <= 1 ? 1 : (K <= 2 ? 2 : (K <= 4 ? 4 : 8));
#define L4(C, GV, M, F)                                                                      \
  hipLaunchKernelGGL((finalize_kernel<C, GV, M, F>), grid, block, 0, stream, y, rows, w,      \
                     row_of_pair, shared, gamma, eps, T, K, D, flags, out, mx_codes, mx_scales)
#define L3(C, GV)                        \
  do {                                   \
    if (mx && full) L4(C, GV, true, true);       \
    else if (mx) L4(C, GV, true, false);         \
    else if (full) L4(C, GV, false, true);       \
    else L4(C, GV, false, false);                \
  } while (0)
#define L(C)                                                  \
  do {                                                        \
    constexpr int gmax = 16 / (C) < 8 ? 16 / (C) : 8;         \
    const int g = gk < gmax ? gk : gmax;                      \
    if (g == 1) L3(C, 1);                                     \
    else if (g == 2) L3(C, (gmax >= 2 ? 2 : 1));              \
    else if (g == 4) L3(C, (gmax >= 4 ? 4 : 1));              \
    else L3(C, (gmax >= 8 ? 8 : 1));                          \
  } while (0)
  switch (sh.cpl) {
    case 1: L(1); break;
    case 2: L(2); break;
    case 4: L(4); break;
    default: L(8); break;
  }
#undef L
#undef L3
#undef L4
  return hipGetLastError();
}

hipError_t launch_finalize_mhc(const uint16_t* y, int64_t rows, const void* w,
                               const int* row_of_pair, const uint16_t* shared,
                               const uint16_t* residual, const float* post, const float* comb,
                               const float* pre, const uint16_t* gamma, float eps, int T, int K,
                               int D, int hc, uint32_t flags, uint16_t* residual_out,
                               uint16_t* out, uint8_t* mx_codes, uint8_t* mx_scales,
                               hipStream_t stream) {
  // one chunk per lane where the row fits 16 waves (the hc streams take
  // registers), else two or four
  const int nch = D / kChunk;
  static const int allowed[] = {1, 2, 4};
  const SliceShape sh = pick_slices(nch, allowed, 3, kMaxWaves);
  const bool norm = pre != nullptr;
  const bool mx = norm && mx_codes != nullptr;
  const int pad_rows = (mx && (flags & 4u)) ? (T + 127) / 128 * 128 - T : 0;
  const dim3 grid(static_cast<unsigned>(T + pad_rows));
  const dim3 block(sh.nsl * kWave);
  const bool full = sh.nsl * kWave * sh.cpl == nch;
  // rows in flight per group: as for the plain finalize, with G * cpl <= 8
  // (the hc residual streams hold registers too)
  const int gk = K <= 1 ? 1 : (K <= 2 ? 2 : (K <= 4 ? 4 : 8));
#define L6(C, GV, H, M, F, N)                                                                 \
  hipLaunchKernelGGL((finalize_mhc_kernel<C, GV, H, M, F, N>), grid, block, 0, stream, y,     \
                     rows, w, row_of_pair, shared, residual, post, comb, pre, gamma, eps, T, K, \
                     D, flags, residual_out, out, mx_codes, mx_scales)
#define L5(C, GV, H)                                \
  do {                                              \
    if (!norm && full) L6(C, GV, H, false, true, false);  \
    else if (!norm) L6(C, GV, H, false, false, false);    \
    else if (mx && full) L6(C, GV, H, true, true, true);  \
    else if (mx) L6(C, GV, H, true, false, true);         \
    else if (full) L6(C, GV, H, false, true, true);       \
    else L6(C, GV, H, false, false, true);                \
  } while (0)
#define L4(C, GV)                    \
  do {                               \
    switch (hc) {                    \
      case 1: L5(C, GV, 1); break;   \
      case 2: L5(C, GV, 2); break;   \
      case 3: L5(C, GV, 3); break;   \
      default: L5(C, GV, 4); break;  \
    }                                \
  } while (0)
#define L(C)                                                  \
  do {                                                        \
    constexpr int gmax = 8 / (C);                             \
    const int g = gk < gmax ? gk : gmax;                      \
    if (g == 1) L4(C, 1);                                     \
    else if (g == 2) L4(C, 2);                                \
    else if (g == 4) L4(C, (gmax >= 4 ? 4 : 2));              \
    else L4(C, (gmax >= 8 ? 8 : 2));                          \
  } while (0)
  switch (sh.cpl) {
    case 1: L(1); break;
    case 2: L(2); break;
    default: L(4); break;
  }
#undef L
#undef L4
#undef L5
#undef L6
  return hipGetLastError();
}

hipError_t launch_convert_check(const float* in, int64_t n, uint16_t* bf16_out,
                                uint8_t* e4m3_out, hipStream_t stream) {
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(convert_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     in, n, bf16_out, e4m3_out);
  return hipGetLastError();
}

}  // namespace moe
