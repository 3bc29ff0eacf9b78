// moe_shuffle: top-k routing and the stable counting sort of the
// (token, expert) pairs by expert, as three launches with no global atomics:
//
//  1. select_rank  (one block per 64 tokens, 16 waves): each wave takes the
//     top-k of a token with the expert axis spread over its 64 lanes (K rounds
//     of a wave-wide max over 64-bit keys that order by score, then by lower
//     expert id). The block then ORs one bit per token into a 64-bit LDS mask
//     per expert; a pair's rank inside its block and expert is the popcount
//     of the mask bits of the tokens before it, and the block's per-expert
//     count is the mask's popcount. Writes (expert | rank << 16) per pair and
//     the [E][blocks] histogram.
//  2. scan  (one block): exclusive scan of the histogram in expert-major
//     order gives every (expert, block) its first row; counts[] follow.
//  3. place  (one thread per pair): row = offset[expert][block] + rank;
//     writes token_indices, expert_indices, row_of_pair. Pairs of tokens at
//     or beyond the valid count keep their natural position t*K + k, which is
//     exactly the tail order (t, k) after the V valid rows.
//
// [LY] "mslk/moe/layers.py", MetaShufflingMoE._route (index shuffling of the
// router scores, per-expert counts) and BaselineMoE._forward (top-k routing).
#include "device.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kTokPerBlock = 64;   // one bit per token in a 64-bit mask
constexpr int kSelThreads = 1024;  // 16 waves, 4 tokens each
constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;
constexpr int kScanThreads = 1024;

// Larger key = larger score; equal scores: lower expert id. -0 is folded
// into +0 so that the two tie, as IEEE comparison says they are equal.
__device__ __forceinline__ uint64_t topk_key(float s, int e) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(u) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
}

__device__ __forceinline__ int clamp_count(const int* p, int hi) {
  if (!p) return hi;
  int v = *p;
  return v < 0 ? 0 : (v > hi ? hi : v);
}

// PL = expert candidates per lane (E <= 64 * PL).
template <int PL>
__global__ __launch_bounds__(kSelThreads) void select_rank_kernel(
    const float* __restrict__ scores, int64_t st, int64_t se, int T, int E, int K,
    const int* __restrict__ vtc_ptr, int* __restrict__ pair, int* __restrict__ hist,
    int nblk) {
  __shared__ unsigned long long mask[kMaxE];
  __shared__ int sel[kTokPerBlock * kMaxK];

  const int blk = blockIdx.x;
  const int t0 = blk * kTokPerBlock;
  const int vtc = clamp_count(vtc_ptr, T);
  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int nwaves = kSelThreads / kWave;

  for (int e = threadIdx.x; e < E; e += kSelThreads) mask[e] = 0ull;

  // ---- top-k, one token per wave at a time
  for (int tl = wave; tl < kTokPerBlock; tl += nwaves) {
    const int t = t0 + tl;
    if (t >= vtc) break;
    const float* srow = scores + static_cast<int64_t>(t) * st;
    uint64_t key[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int e = j * kWave + lane;
      key[j] = (e < E) ? topk_key(srow[static_cast<int64_t>(e) * se], e) : 0ull;
    }
    for (int k = 0; k < K; ++k) {
      uint64_t best = key[0];
#pragma unroll
      for (int j = 1; j < PL; ++j) best = key[j] > best ? key[j] : best;
      const uint64_t win = wave_max_u64(best);
#pragma unroll
      for (int j = 0; j < PL; ++j)
        if (key[j] == win) key[j] = 0ull;  // keys are unique: one owner
      if (lane == 0)
        sel[tl * K + k] = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(win));
    }
  }
  __syncthreads();

  // ---- one bit per valid token in each of its experts' masks
  const int npairs = kTokPerBlock * K;
  for (int p = threadIdx.x; p < npairs; p += kSelThreads) {
    const int tl = p / K;
    if (t0 + tl < vtc) atomicOr(&mask[sel[p]], 1ull << tl);
  }
  __syncthreads();

  // ---- stable rank inside (block, expert) and the block histogram
  for (int p = threadIdx.x; p < npairs; p += kSelThreads) {
    const int tl = p / K;
    const int t = t0 + tl;
    if (t < vtc) {
      const int e = sel[p];
      const unsigned long long before = mask[e] & ((1ull << tl) - 1ull);
      pair[static_cast<int64_t>(t0) * K + p] = e | (__popcll(before) << 16);
    }
  }
  for (int e = threadIdx.x; e < E; e += kSelThreads)
    hist[static_cast<int64_t>(e) * nblk + blk] = __popcll(mask[e]);
}

// Exclusive scan of hist[E*nblk] (expert-major) in place; counts[e] is the
// row length of expert e, counts[E] the total.
__global__ __launch_bounds__(kScanThreads) void scan_kernel(int* __restrict__ hist, int E,
                                                            int nblk,
                                                            int* __restrict__ counts) {
  __shared__ int part[kScanThreads];
  __shared__ int row_start[kMaxE + 1];
  const int n = E * nblk;
  const int tid = threadIdx.x;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int beg = min(tid * per, n);
  const int end = min(beg + per, n);
  for (int e = tid; e <= E; e += kScanThreads) row_start[e] = 0;

  int s = 0;
  for (int i = beg; i < end; ++i) s += hist[i];
  part[tid] = s;
  __syncthreads();
  // Hillis-Steele inclusive scan of the per-thread sums
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;  // exclusive prefix
  for (int i = beg; i < end; ++i) {
    const int c = hist[i];
    if (i % nblk == 0) row_start[i / nblk] = run;  // nblk > 0 here
    hist[i] = run;
    run += c;
  }
  __syncthreads();
  if (tid == kScanThreads - 1) row_start[E] = part[tid];
  __syncthreads();
  for (int e = tid; e < E; e += kScanThreads) counts[e] = row_start[e + 1] - row_start[e];
  if (tid == 0) counts[E] = row_start[E];
}

__global__ __launch_bounds__(256) void place_kernel(const int* __restrict__ pair,
                                                    const int* __restrict__ offs, int nblk,
                                                    int T, int K,
                                                    const int* __restrict__ vtc_ptr,
                                                    int* __restrict__ ti, int* __restrict__ ei,
                                                    int* __restrict__ rop) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t npairs = static_cast<int64_t>(T) * K;
  if (p >= npairs) return;
  const int t = static_cast<int>(p / K);
  const int vtc = clamp_count(vtc_ptr, T);
  if (t < vtc) {
    const int v = pair[p];
    const int e = v & 0xFFFF;
    const int rank = v >> 16;
    const int r = offs[static_cast<int64_t>(e) * nblk + t / kTokPerBlock] + rank;
    ti[r] = t;
    ei[r] = e;
    if (rop) rop[p] = r;
  } else {
    ti[p] = t;
    ei[p] = -1;
    if (rop) rop[p] = -1;
  }
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

}  // namespace

size_t shuffle_workspace_bytes(int T, int E, int K) {
  const int nblk = (T + kTokPerBlock - 1) / kTokPerBlock;
  return align256(static_cast<size_t>(T) * K * sizeof(int)) +
         align256(static_cast<size_t>(E) * nblk * sizeof(int));
}

hipError_t launch_shuffle(const float* scores, int64_t st, int64_t se, int T, int E,
                          int K, const int* vtc, int* counts, int* expert_indices,
                          int* token_indices, int* row_of_pair, void* workspace,
                          hipStream_t stream) {
  const int nblk = (T + kTokPerBlock - 1) / kTokPerBlock;
  char* ws = static_cast<char*>(workspace);
  int* pair = reinterpret_cast<int*>(ws);
  int* hist = reinterpret_cast<int*>(ws + align256(static_cast<size_t>(T) * K * sizeof(int)));
  if (T == 0) {
    // no pairs: every count is zero
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, hist, E, 0,
                       counts);
    return hipGetLastError();
  }
  const int pl = (E + kWave - 1) / kWave;
  const dim3 g1(nblk), b1(kSelThreads);
#define MOE_SEL(PLV)                                                                     \
  hipLaunchKernelGGL(select_rank_kernel<PLV>, g1, b1, 0, stream, scores, st, se, T, E, K, \
                     vtc, pair, hist, nblk)
  if (pl <= 1) MOE_SEL(1);
  else if (pl <= 2) MOE_SEL(2);
  else if (pl <= 4) MOE_SEL(4);
  else if (pl <= 8) MOE_SEL(8);
  else MOE_SEL(16);
#undef MOE_SEL
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, hist, E, nblk,
                     counts);
  const int64_t npairs = static_cast<int64_t>(T) * K;
  const int pblocks = static_cast<int>((npairs + 255) / 256);
  hipLaunchKernelGGL(place_kernel, dim3(pblocks), dim3(256), 0, stream, pair, hist, nblk, T,
                     K, vtc, token_indices, expert_indices, row_of_pair);
  return hipGetLastError();
}

}  // namespace moe
