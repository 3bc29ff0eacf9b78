// Device helpers shared by the gfx950 kernels: 16-byte vector memory access,
// bf16 / E4M3 conversion, wave64 reductions and the row-slice layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kChunk = 8;  // bf16 elements per 16-byte vector ("chunk")

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- memory
// Plain 16-byte loads go through L2 (reused data: gathered token rows).
__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// Streaming data (read once): non-temporal hint, so it does not displace
// reused lines.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}
// Output rows are written once and not read back by this kernel.
__device__ __forceinline__ void st16_stream(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st8_stream(void* p, u32x2 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x2*>(p));
}

// ---------------------------------------------------------------- bf16
// Widening bf16 -> fp32 is exact: the bf16 bits are the upper half.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 round-to-nearest-even, two at a time (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v.x = static_cast<__bf16>(lo);
  v.y = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ void unpack8(u32x4 v, float f[8]) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}
__device__ __forceinline__ u32x4 pack8(const float f[8]) {
  u32x4 v;
  v.x = pack_bf16x2(f[0], f[1]);
  v.y = pack_bf16x2(f[2], f[3]);
  v.z = pack_bf16x2(f[4], f[5]);
  v.w = pack_bf16x2(f[6], f[7]);
  return v;
}

// ---------------------------------------------------------------- E4M3
// fp32 -> OCP E4M3FN, round to nearest even (v_cvt_pk_fp8_f32; gfx950 uses
// the OCP encoding). Callers clamp to [-448, 448] first.
constexpr float kE4M3Max = 448.0f;
__device__ __forceinline__ float clamp448(float v) {
  return __builtin_fminf(__builtin_fmaxf(v, -kE4M3Max), kE4M3Max);
}
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return static_cast<uint32_t>(w);
}

// ---------------------------------------------------------------- reductions
// The value a DPP lane move brings to each lane (CTRL selects the source
// lane); lanes of rows outside ROW_MASK get `identity` instead.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_from(float v, float identity) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(v),
                                                    CTRL, ROW_MASK, 0xF, false));
}

// Wave-wide sum and max by DPP lane moves, no LDS-pipe round trips. Quad
// swaps and the half-row and row mirrors leave each 16-lane row's result in
// all its lanes; row_bcast15 then folds row 0 into row 1 and row 2 into row
// 3, row_bcast31 row 1 into row 3, whose lane 63 holds the wave's result
// (returned to every lane). Every lane of the wave must be active.
__device__ __forceinline__ float wave_sum(float v) {
  v = v + dpp_from<0xB1, 0xF>(v, -0.0f);   // quad_perm [1,0,3,2]
  v = v + dpp_from<0x4E, 0xF>(v, -0.0f);   // quad_perm [2,3,0,1]
  v = v + dpp_from<0x141, 0xF>(v, -0.0f);  // row_half_mirror
  v = v + dpp_from<0x140, 0xF>(v, -0.0f);  // row_mirror
  v = v + dpp_from<0x142, 0xA>(v, -0.0f);  // row_bcast15 into rows 1 and 3
  v = v + dpp_from<0x143, 0xC>(v, -0.0f);  // row_bcast31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// The same sum in fp64: each DPP step moves the two 32-bit halves of the
// double with the same control (lanes of masked rows get -0.0).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_from_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_update_dpp(0, static_cast<int>(u & 0xFFFFFFFFu), CTRL,
                                             ROW_MASK, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(static_cast<int>(0x80000000u),
                                             static_cast<int>(u >> 32), CTRL, ROW_MASK, 0xF,
                                             false);
  return __builtin_bit_cast(double, (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                        static_cast<uint32_t>(lo));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = v + dpp_from_f64<0xB1, 0xF>(v);
  v = v + dpp_from_f64<0x4E, 0xF>(v);
  v = v + dpp_from_f64<0x141, 0xF>(v);
  v = v + dpp_from_f64<0x140, 0xF>(v);
  v = v + dpp_from_f64<0x142, 0xA>(v);
  v = v + dpp_from_f64<0x143, 0xC>(v);
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = static_cast<uint32_t>(
      __builtin_amdgcn_readlane(static_cast<int>(u & 0xFFFFFFFFu), 63));
  const uint32_t hi =
      static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u >> 32), 63));
  return __builtin_bit_cast(double, (static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ float wave_max(float v) {
  const float lo = -__builtin_inff();
  v = __builtin_fmaxf(v, dpp_from<0xB1, 0xF>(v, lo));
  v = __builtin_fmaxf(v, dpp_from<0x4E, 0xF>(v, lo));
  v = __builtin_fmaxf(v, dpp_from<0x141, 0xF>(v, lo));
  v = __builtin_fmaxf(v, dpp_from<0x140, 0xF>(v, lo));
  v = __builtin_fmaxf(v, dpp_from<0x142, 0xA>(v, lo));
  v = __builtin_fmaxf(v, dpp_from<0x143, 0xC>(v, lo));
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Uniform (scalar) copy of a wave-uniform value.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Number of set bits of m below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0));
}

// The rows r < V with token index t, found by the wave itself: tv[c] holds
// token_indices[64c + lane] (-1 from V on). Chunk by chunk a ballot marks the
// token's rows, which are staged in this wave's 64 LDS words in ascending
// order and handed to batch(rows, n) up to 64 at a time (lane i of `rows`
// holds the batch's i-th row; lanes from n on hold no row). Returns the
// number of rows. V and t are wave-uniform.
template <int NC, class F>
__device__ __forceinline__ int for_token_rows(const int (&tv)[NC], int V, int t, int lane,
                                              int* __restrict__ stage, F&& batch) {
  int cnt = 0;
  int total = 0;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    if (c * kWave >= V) break;
    const bool hit = tv[c] == t;
    const uint64_t m = __ballot(hit);
    const int nb = __popcll(m);
    if (nb == 0) continue;
    if (cnt + nb > kWave) {
      batch(stage[lane], cnt);
      cnt = 0;
    }
    if (hit) stage[cnt + lanes_below(m)] = c * kWave + lane;
    cnt += nb;
    total += nb;
  }
  if (cnt) batch(stage[lane], cnt);
  return total;
}

}  // namespace moe
