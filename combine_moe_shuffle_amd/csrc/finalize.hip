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

// FULL: every wave's slice lies inside the row (D == waves * 64 * CPL * 8),
// so no chunk needs a bounds test and loads/stores are straight-line code.
// G: expert rows in flight per group (>= K where possible: one group).
template <int CPL, int G, bool MX, bool FULL>
__global__ __launch_bounds__(kMaxWaves* kWave) void finalize_kernel(
    const uint16_t* __restrict__ y, int64_t rows, const float* __restrict__ w,
    const int* __restrict__ rop, const uint16_t* __restrict__ shared,
    const uint16_t* __restrict__ gamma, float eps, int K, int D, uint32_t flags,
    uint16_t* __restrict__ out, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  __shared__ float wave_ss[kMaxWaves];

  const int t = blockIdx.x;
  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int nch = D >> 3;
  const int base = wave * kWave * CPL + lane;

  // lane k holds slot k (K <= 64): its row (or -1) and weight
  int my_r = -1;
  float my_w = 0.0f;
  if (lane < K) {
    my_r = rop[static_cast<int64_t>(t) * K + lane];
    my_w = w[static_cast<int64_t>(t) * K + lane];
    if (my_r >= rows) my_r = -1;  // out of range: treated as not held
  }

  float acc[CPL][8];
#pragma unroll
  for (int j = 0; j < CPL; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = 0.0f;

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

  // h = bf16(acc [+ shared]); keep h as packed bf16 and its square sum
  u32x4 h[CPL];
  float ss = 0.0f;
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = base + j * kWave;
    if (FULL || c < nch) {
      if (shared) {
        float f[8];
        unpack8(sh[j], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[j][i] = acc[j][i] + f[i];
      }
      h[j] = pack8(acc[j]);
      float hf[8];
      unpack8(h[j], hf);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float sq = hf[i] * hf[i];
        if (flags & 1u) sq = bf16_lo(pack_bf16x2(sq, 0.0f));
        ss = ss + sq;
      }
    }
  }
  ss = wave_sum(ss);
  if (lane == 0) wave_ss[wave] = ss;
  __syncthreads();
  float total = 0.0f;
  for (int v = 0; v < nwaves; ++v) total = total + wave_ss[v];
  const float mean = total / static_cast<float>(D);
  const float inv = static_cast<float>(1.0 / sqrt(static_cast<double>(mean + eps)));

  uint16_t* orow = out + static_cast<int64_t>(t) * D;
  u32x4 ob[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    float hf[8], g[8], o[8];
    unpack8(h[j], hf);
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
        if ((lane & 3) == 0)
          scales[static_cast<int64_t>(t) * (D >> 5) + (c >> 2)] = static_cast<uint8_t>(bytes[j]);
      }
    }
  }
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

hipError_t launch_finalize_rmsnorm(const uint16_t* y, int64_t rows, const float* w,
                                   const int* row_of_pair, const uint16_t* shared,
                                   const uint16_t* gamma, float eps, int T, int K, int D,
                                   uint32_t flags, uint16_t* out, uint8_t* mx_codes,
                                   uint8_t* mx_scales, hipStream_t stream) {
  // few tokens: one chunk per lane and up to 16 waves per token (latency);
  // many tokens: two chunks per lane, fewer waves per token
  const int nch = D / kChunk;
  static const int small_t[] = {1, 2, 4, 8};
  static const int large_t[] = {2, 4, 8, 1};
  const SliceShape sh = T < 2048 ? pick_slices(nch, small_t, 4, kMaxWaves)
                                  : pick_slices(nch, large_t, 4, kMaxWaves);
  const dim3 grid(static_cast<unsigned>(T));
  const dim3 block(sh.nsl * kWave);
  const bool mx = mx_codes != nullptr;
  const bool full = sh.nsl * kWave * sh.cpl == nch;
  // rows in flight per group: the next power of two >= K (at most 8), with
  // G * cpl <= 16 to bound the registers
  const int gk = K <= 1 ? 1 : (K <= 2 ? 2 : (K <= 4 ? 4 : 8));
#define L4(C, GV, M, F)                                                                      \
  hipLaunchKernelGGL((finalize_kernel<C, GV, M, F>), grid, block, 0, stream, y, rows, w,      \
                     row_of_pair, shared, gamma, eps, K, D, flags, out, mx_codes, mx_scales)
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

hipError_t launch_convert_check(const float* in, int64_t n, uint16_t* bf16_out,
                                uint8_t* e4m3_out, hipStream_t stream) {
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(convert_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     in, n, bf16_out, e4m3_out);
  return hipGetLastError();
}

}  // namespace moe
