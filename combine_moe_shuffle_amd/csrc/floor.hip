// Latency floors of the finalize's launch: kernels with the finalize's grid
// and workgroup shape for (T, D) that do (0) nothing, or (1) two dependent
// 16-byte loads per lane (an index, then the element it points at) and one
// store. Timed beside the finalize they bound what a one-token-per-workgroup
// kernel can reach at small T: the launch itself, and the two memory round
// trips the finalize's slot rows and expert rows take.
#include "device.hpp"
#include "launch.hpp"

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

}  // namespace moe
