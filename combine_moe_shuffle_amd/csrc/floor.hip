// Measurement aids, timed beside the path's kernels and used by none of them.
//
// Latency floors of the finalize's launch: kernels with the finalize's grid
// and workgroup shape for (T, D) that do (0) nothing, or (1) two dependent
// 16-byte loads per lane (an index, then the element it points at) and one
// store. Timed beside the finalize they bound what a one-token-per-workgroup
// kernel can reach at small T: the launch itself, and the two memory round
// trips the finalize's slot rows and expert rows take.
//
// A contiguous stream with a chosen read:write mix, in one of two layouts:
// blocked (wave u reads R consecutive KiB of src and writes W consecutive KiB
// of dst, consecutive waves on consecutive memory) or interleaved (src is R
// streams and dst W streams of `units` KiB each; wave u reads and writes KiB
// u of every stream, consecutive waves on consecutive memory in each). Every
// access is a nontemporal 16-byte one per lane, as in the streaming kernels.
// Few streams favour the interleaved layout, many streams the blocked one.
// Timed with a streaming kernel's byte counts it gives a reference rate for
// that mix: what a plain stream of the same bytes reaches, next to the HBM
// peak.
#include "device.hpp"
#include "launch.hpp"
#include "probe.hpp"

namespace moe {

namespace {

__global__ void floor_empty_kernel() {}

__global__ __launch_bounds__(1024) void floor_loads_kernel(const u32x4* __restrict__ src,
                                                           int* __restrict__ dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const u32x4 a = src[i];
  const u32x4 b = src[a.x % static_cast<uint32_t>(n)];
  dst[i] = static_cast<int>(b.x + b.y + b.z + b.w);
}

constexpr int kProbeWaves = 4;

// Each 16-byte word written is the wrapping uint32 sum, lane by lane, of the
// R words at the same position of the wave's R source KiB, xor the index
// (0..W-1) of the destination KiB it lands in (blocked: the wave's w-th KiB;
// interleaved: stream w).
template <int R, bool INTERLEAVED>
__global__ __launch_bounds__(kProbeWaves* kWave) void stream_probe_kernel(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, int W, int64_t units) {
  const int64_t u = static_cast<int64_t>(blockIdx.x) * kProbeWaves + (threadIdx.x >> 6);
  if (u >= units) return;
  const int lane = lane_id();
  constexpr int kWordsPerKiB = 1024 / 16;
  // distance between a wave's consecutive KiB, and the wave's first KiB
  const int64_t rstep = INTERLEAVED ? units * kWordsPerKiB : kWordsPerKiB;
  const int64_t wstep = rstep;
  const u32x4* s = src + (INTERLEAVED ? u : u * R) * kWordsPerKiB + lane;
  u32x4* d = dst + (INTERLEAVED ? u : u * W) * kWordsPerKiB + lane;
  u32x4 v[R];
#pragma unroll
  for (int r = 0; r < R; ++r) v[r] = ld16_stream(s + r * rstep);
  u32x4 acc = v[0];
#pragma unroll
  for (int r = 1; r < R; ++r) acc += v[r];
  for (int w = 0; w < W; ++w) st16_stream(d + w * wstep, acc ^ static_cast<uint32_t>(w));
}

}  // namespace

SliceShape finalize_launch_shape(int T, int D);

int launch_floor_threads(int T, int D) { return finalize_launch_shape(T, D).nsl * kWave; }

hipError_t launch_floor(int kind, int T, int D, const void* src, void* dst,
                        hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(T));
  const dim3 block(static_cast<unsigned>(launch_floor_threads(T, D)));
  if (kind == 0) {
    hipLaunchKernelGGL(floor_empty_kernel, grid, block, 0, stream);
  } else {
    hipLaunchKernelGGL(floor_loads_kernel, grid, block, 0, stream,
                       static_cast<const u32x4*>(src), static_cast<int*>(dst),
                       static_cast<int>(grid.x * block.x));
  }
  return hipGetLastError();
}

hipError_t launch_stream_probe(int layout, int R, int W, int64_t units, const void* src,
                               void* dst, hipStream_t stream) {
  if (units <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((units + kProbeWaves - 1) / kProbeWaves));
  const dim3 block(kProbeWaves * kWave);
  const u32x4* s = static_cast<const u32x4*>(src);
  u32x4* d = static_cast<u32x4*>(dst);
  static_assert(kStreamMaxR == 32, "one case below for every R in [1, kStreamMaxR]");
  switch (R) {
#define MOE_PROBE_CASE(RV)                                                                     \
  case RV:                                                                                     \
    if (layout == 1)                                                                           \
      hipLaunchKernelGGL((stream_probe_kernel<RV, true>), grid, block, 0, stream, s, d, W,     \
                         units);                                                               \
    else                                                                                       \
      hipLaunchKernelGGL((stream_probe_kernel<RV, false>), grid, block, 0, stream, s, d, W,    \
                         units);                                                               \
    break;
    MOE_PROBE_CASE(1) MOE_PROBE_CASE(2) MOE_PROBE_CASE(3) MOE_PROBE_CASE(4)
    MOE_PROBE_CASE(5) MOE_PROBE_CASE(6) MOE_PROBE_CASE(7) MOE_PROBE_CASE(8)
    MOE_PROBE_CASE(9) MOE_PROBE_CASE(10) MOE_PROBE_CASE(11) MOE_PROBE_CASE(12)
    MOE_PROBE_CASE(13) MOE_PROBE_CASE(14) MOE_PROBE_CASE(15) MOE_PROBE_CASE(16)
    MOE_PROBE_CASE(17) MOE_PROBE_CASE(18) MOE_PROBE_CASE(19) MOE_PROBE_CASE(20)
    MOE_PROBE_CASE(21) MOE_PROBE_CASE(22) MOE_PROBE_CASE(23) MOE_PROBE_CASE(24)
    MOE_PROBE_CASE(25) MOE_PROBE_CASE(26) MOE_PROBE_CASE(27) MOE_PROBE_CASE(28)
    MOE_PROBE_CASE(29) MOE_PROBE_CASE(30) MOE_PROBE_CASE(31) MOE_PROBE_CASE(32)
#undef MOE_PROBE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
