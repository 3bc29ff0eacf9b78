// Expert-parallel receive-side re-sort (combine_shuffling) and its inverse
// (split_shuffling).
//
// [LY] "mslk/moe/layers.py", _dynamic_comm_forward and _static_comm_forward:
// rows received from EP ranks arrive grouped by source rank, and inside a
// rank's chunk by expert column; the expert GEMMs need them grouped by local
// expert, and the results go back in the received order. Segment (r, c) holds
// counts[r*C + c] rows; rank r's chunk starts at r * rank_stride, or right
// after rank r-1's chunk when rank_stride < 0 (packed). The local columns
// [c_lo, c_hi) are gathered expert-major: for each local column, the segments
// of ranks 0..EP-1 in turn.
//
// Three launches: one workgroup builds the segment table (per-rank column
// scans, rank bases, and the expert-major scan, in LDS); one wave per segment
// writes every expert-major row's rank-major row; then one wave per (row,
// slice) copies the row with 16-byte loads and stores, one table load ahead
// of its row.
#include <limits.h>

#include "device.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kTableThreads = 1024;
constexpr int kScanPer = kMaxShufflingSegments / kTableThreads;  // 4
constexpr int kRowWaves = 4;

// seg_src[q] / seg_dst[q]: first rank-major / expert-major row of segment
// q = l*EP + r (l = local column); seg_dst[nseg] = total rows;
// out_counts[l] = rows of local column l, out_counts[nl] = total.
__global__ __launch_bounds__(kTableThreads) void shuffling_table_kernel(
    const int* __restrict__ counts, int EP, int C, int c_lo, int c_hi, int64_t rank_stride,
    int* __restrict__ seg_src, int* __restrict__ seg_dst, int* __restrict__ out_counts) {
  __shared__ int cnt[kMaxShufflingSegments];
  __shared__ int off[kMaxShufflingSegments];
  __shared__ int rank_total[kMaxShufflingRanks];
  __shared__ int base[kMaxShufflingRanks];
  __shared__ int wave_tot[kTableThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int nl = c_hi - c_lo;
  const int nseg = nl * EP;

  // 1. per rank: exclusive scan over its C columns (one wave per rank)
  for (int r = wave; r < EP; r += kTableThreads / kWave) {
    int carry = 0;
    for (int c0 = 0; c0 < C; c0 += kWave) {
      const int c = c0 + lane;
      const int v = c < C ? max(counts[static_cast<int64_t>(r) * C + c], 0) : 0;
      int incl = v;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int u = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += u;
      }
      if (c >= c_lo && c < c_hi) {
        const int q = (c - c_lo) * EP + r;
        off[q] = carry + incl - v;
        cnt[q] = v;
      }
      carry += __shfl(incl, kWave - 1, kWave);
    }
    if (lane == 0) rank_total[r] = carry;
  }
  __syncthreads();
  // 2. rank bases (EP <= 64: one wave)
  if (wave == 0) {
    const int v = lane < EP ? rank_total[lane] : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int u = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += u;
    }
    if (lane < EP)
      base[lane] = rank_stride >= 0 ? static_cast<int>(lane * rank_stride) : incl - v;
  }
  __syncthreads();
  // 3. expert-major exclusive scan of the segment sizes; thread tid owns
  //    segments tid*kScanPer .. tid*kScanPer + kScanPer - 1
  int v[kScanPer];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    const int q = tid * kScanPer + i;
    v[i] = q < nseg ? cnt[q] : 0;
    mine += v[i];
  }
  int incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int run = incl - mine, total = 0;
  for (int w = 0; w < kTableThreads / kWave; ++w) {
    if (w < wave) run += wave_tot[w];
    total += wave_tot[w];
  }
#pragma unroll
  for (int i = 0; i < kScanPer; ++i) {
    const int q = tid * kScanPer + i;
    if (q < nseg) {
      seg_dst[q] = run;
      seg_src[q] = base[q % EP] + off[q];
      cnt[q] = run;  // reuse: expert-major start, read back below
    }
    run += v[i];
  }
  __syncthreads();
  if (tid == 0) seg_dst[nseg] = total;
  if (!out_counts) return;
  if (tid == 0) out_counts[nl] = total;
  for (int l = tid; l < nl; l += kTableThreads) {
    const int s0 = cnt[l * EP];
    const int s1 = l + 1 < nl ? cnt[(l + 1) * EP] : total;
    out_counts[l] = s1 - s0;
  }
}

// src_of_row[o] = the rank-major row of expert-major row o: segment q's
// rank-major start plus o's offset in the segment (one wave per segment).
// Rows are taken in 64 bits and only rows in [0, em_rows) are written, so
// counts whose sums pass 2^31 - 1 (wrapped table entries) write nothing out
// of range; an entry past INT_MAX is stored as INT_MAX, which the copy drops. Rows at or beyond em_rows (counts larger than the buffer) are not
// marked; the copy kernel never reaches them.
__global__ __launch_bounds__(kRowWaves* kWave) void shuffling_mark_kernel(
    const int* __restrict__ seg_src, const int* __restrict__ seg_dst, int nseg,
    int64_t em_rows, int* __restrict__ src_of_row) {
  const int q = blockIdx.x * kRowWaves + uniform(threadIdx.x >> 6);
  if (q >= nseg) return;
  const int s0 = seg_dst[q];
  const int len = seg_dst[q + 1] - s0;
  const int r0 = seg_src[q];
  for (int j = lane_id(); j < len; j += kWave) {
    const int64_t o = static_cast<int64_t>(s0) + j;
    const int64_t r = static_cast<int64_t>(r0) + j;
    if (o >= 0 && o < em_rows) src_of_row[o] = r > INT_MAX ? INT_MAX : static_cast<int>(r);
  }
}

// Copies expert-major row o from / to its rank-major position.
// INVERSE = false (combine): out[o] = in[src(o)]; true (split): out[src(o)] = in[o].
template <int CPL, bool INVERSE>
__global__ __launch_bounds__(kRowWaves* kWave) void shuffling_copy_kernel(
    const uint16_t* __restrict__ in, int64_t in_rows, uint16_t* __restrict__ out,
    int64_t out_rows, int D, const int* __restrict__ seg_dst, int nseg,
    const int* __restrict__ src_of_row, int64_t em_rows, int nsl) {
  const int lane = lane_id();
  const int64_t unit =
      static_cast<int64_t>(blockIdx.x) * kRowWaves + uniform(threadIdx.x >> 6);
  const int64_t o = unit / nsl;
  const int sl = static_cast<int>(unit - o * nsl);
  if (o >= em_rows) return;
  // both loads at once; rows at or past the total were not written by the
  // mark kernel and are dropped before their entry is used
  const int total = seg_dst[nseg];
  const int64_t rm = src_of_row[o];
  if (o >= total) return;
  const int64_t from = INVERSE ? o : rm;
  const int64_t to = INVERSE ? rm : o;
  // out-of-range layout (a negative row only from wrapped counts): skipped
  if (rm < 0 || from >= in_rows || to >= out_rows) return;
  const uint16_t* src = in + from * D;
  uint16_t* dst = out + to * D;
  const int nch = D >> 3;
  const int slice0 = sl * kWave * CPL;
  const int base = slice0 + lane;
  u32x4 v[CPL];
  if (slice0 + kWave * CPL <= nch) {
#pragma unroll
    for (int j = 0; j < CPL; ++j) v[j] = ld16_stream(src + (base + j * kWave) * kChunk);
#pragma unroll
    for (int j = 0; j < CPL; ++j) st16_stream(dst + (base + j * kWave) * kChunk, v[j]);
  } else {
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = base + j * kWave;
      if (c < nch) v[j] = ld16_stream(src + c * kChunk);
    }
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = base + j * kWave;
      if (c < nch) st16_stream(dst + c * kChunk, v[j]);
    }
  }
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

}  // namespace

size_t shuffling_workspace_bytes(int nseg, int64_t em_rows) {
  return 2 * align256((static_cast<size_t>(nseg) + 1) * sizeof(int)) +
         align256(static_cast<size_t>(em_rows) * sizeof(int));
}

hipError_t launch_shuffling(bool inverse, const uint16_t* in, int64_t in_rows, uint16_t* out,
                            int64_t out_rows, int D, const int* counts, int EP, int C, int c_lo,
                            int c_hi, int64_t rank_stride, int* out_counts, void* workspace,
                            hipStream_t stream) {
  const int nseg = (c_hi - c_lo) * EP;
  const int64_t em_rows = inverse ? in_rows : out_rows;  // rows of the expert-major side
  char* ws = static_cast<char*>(workspace);
  int* seg_src = reinterpret_cast<int*>(ws);
  int* seg_dst = reinterpret_cast<int*>(ws + align256((static_cast<size_t>(nseg) + 1) * 4));
  int* src_of_row =
      reinterpret_cast<int*>(ws + 2 * align256((static_cast<size_t>(nseg) + 1) * 4));
  hipLaunchKernelGGL(shuffling_table_kernel, dim3(1), dim3(kTableThreads), 0, stream, counts,
                     EP, C, c_lo, c_hi, rank_stride, seg_src, seg_dst, out_counts);
  if (nseg > 0)
    hipLaunchKernelGGL(shuffling_mark_kernel, dim3((nseg + kRowWaves - 1) / kRowWaves),
                       dim3(kRowWaves * kWave), 0, stream, seg_src, seg_dst, nseg, em_rows,
                       src_of_row);
  if (em_rows == 0 || D == 0 || nseg == 0) return hipGetLastError();
  static const int allowed[] = {1, 2, 3, 4, 5, 6, 7, 8};
  const SliceShape sh = pick_slices(D / kChunk, allowed, 8, 1 << 20);
  const int64_t units = em_rows * sh.nsl;
  const dim3 grid(static_cast<unsigned>((units + kRowWaves - 1) / kRowWaves));
  const dim3 block(kRowWaves * kWave);
#define L(C)                                                                                \
  do {                                                                                      \
    if (inverse)                                                                            \
      hipLaunchKernelGGL((shuffling_copy_kernel<C, true>), grid, block, 0, stream, in,      \
                         in_rows, out, out_rows, D, seg_dst, nseg, src_of_row, em_rows,     \
                         sh.nsl);                                                           \
    else                                                                                    \
      hipLaunchKernelGGL((shuffling_copy_kernel<C, false>), grid, block, 0, stream, in,     \
                         in_rows, out, out_rows, D, seg_dst, nseg, src_of_row, em_rows,     \
                         sh.nsl);                                                           \
  } while (0)
  MOE_DISPATCH_CPL(sh.cpl, L)
#undef L
  return hipGetLastError();
}

}  // namespace moe
