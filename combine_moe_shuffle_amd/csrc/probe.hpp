// Measurement aids that no kernel of the path uses: declared apart from
// launch.hpp so that adding one leaves the path's headers as they are.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace moe {

// floor.hip: a contiguous stream of R KiB read and W KiB written per wave,
// blocked per wave (layout 0) or interleaved over R + W streams (layout 1)
constexpr int kStreamMaxR = 32;
constexpr int kStreamMaxW = 32;
hipError_t launch_stream_probe(int layout, int R, int W, int64_t units, const void* src,
                               void* dst, hipStream_t stream);

}  // namespace moe
