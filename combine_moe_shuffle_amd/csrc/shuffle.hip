// moe_shuffle: top-k routing and the stable counting sort of the
// (token, expert) pairs by expert, as three launches with no global atomics
// (two when the histogram of step 1 fits in LDS: scan_place_kernel does
// steps 2 and 3 in one launch; one for up to 32 tokens, or 64 with short
// top-k rounds, where shuffle_small_kernel does all three in one workgroup):
//
//  1. select_rank  (one workgroup of 16 waves per block of 32 tokens, or of
//     16 tokens for batches of up to 128): each wave takes the top-k of its
//     two tokens (or one) at once, the expert axis spread over its 64 lanes
//     (K rounds of a DPP wave max over order-preserving score keys, the
//     lowest tied lane holding the lowest expert id; two reductions
//     interleave so their lane-exchange latencies overlap). The workgroup
//     then ORs one bit per token into a 32-bit LDS mask per expert; a pair's
//     rank inside its workgroup and expert is the popcount of the mask bits
//     of the tokens before it, the workgroup's per-expert count the mask's
//     popcount.
//     Writes (expert | rank << 16) per pair and the [E][blocks] histogram.
//  2. expert_scan  (one wave per expert): exclusive scan of the expert's row
//     of the histogram over blocks, in place; its total is counts[e].
//  3. place  (one thread per pair): each workgroup scans counts[0..E) in LDS
//     to get every expert's first row, then row = first[e] + offset[e][block]
//     + rank; writes token_indices, expert_indices, row_of_pair. Pairs of
//     tokens at or beyond the valid count keep their natural position
//     t*K + k, which is exactly the tail order (t, k) after the V valid rows.
//
// [LY] "mslk/moe/layers.py", MetaShufflingMoE._route (index shuffling of the
// router scores, per-expert counts) and BaselineMoE._forward (top-k routing).
#include "device.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kTokPerBlock = 32;   // one bit per token in a 32-bit mask
constexpr int kSelThreads = 1024;  // 16 waves, 2 tokens each
constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;

// Order-preserving map of a score to uint32 (larger score -> larger key).
// -0 is folded into +0 so that the two tie, as IEEE comparison says they are
// equal. Every real score maps above 0, which marks an empty candidate.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One DPP max step on N independent values, written step-major so the N
// chains interleave and fill each other's DPP hazard slots.
template <int N, int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_max_step(uint32_t (&v)[N]) {
#pragma unroll
  for (int q = 0; q < N; ++q) {
    if constexpr (ROW_MASK == 0xF) {
      // every lane reads a valid source: the move can fold into the max
      v[q] = max(v[q], static_cast<uint32_t>(__builtin_amdgcn_mov_dpp(
                           static_cast<int>(v[q]), CTRL, 0xF, 0xF, true)));
    } else {
      // lanes of masked rows keep their own value
      v[q] = max(v[q], static_cast<uint32_t>(__builtin_amdgcn_update_dpp(
                           static_cast<int>(v[q]), static_cast<int>(v[q]), CTRL, ROW_MASK,
                           0xF, false)));
    }
  }
}

// Wave-wide max of N uint32 values at once, uniform results. Quad swaps and
// the half-row and row mirrors leave each 16-lane row's max in all its lanes;
// row_bcast15 then folds row 0 into row 1 and row 2 into row 3, row_bcast31
// folds row 1 into rows 2 and 3, so lane 63 holds the wave max.
template <int N>
__device__ __forceinline__ void wave_max_keys(uint32_t (&v)[N], uint32_t (&out)[N]) {
  dpp_max_step<N, 0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  dpp_max_step<N, 0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  dpp_max_step<N, 0x141, 0xF>(v);  // row_half_mirror
  dpp_max_step<N, 0x140, 0xF>(v);  // row_mirror
  dpp_max_step<N, 0x142, 0xA>(v);  // row_bcast15 into rows 1 and 3
  dpp_max_step<N, 0x143, 0xC>(v);  // row_bcast31 into rows 2 and 3
#pragma unroll
  for (int q = 0; q < N; ++q)
    out[q] = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v[q]), 63));
}

__device__ __forceinline__ int clamp_count(const int* p, int hi) {
  if (!p) return hi;
  int v = *p;
  return v < 0 ? 0 : (v > hi ? hi : v);
}

// Top-k of TPW tokens in one wave, worked on together so that their lane
// exchanges overlap: tokens t0 + wave + q * nwaves (q < TPW). Lane l holds
// experts l*PL .. l*PL+PL-1, sorted by (score desc, id asc); a lower lane
// always holds lower ids, so among lanes whose best ties with the wave max the
// lowest lane holds the lowest expert id. Slot k of token i = wave + q *
// nwaves (relative to t0) goes to sel[i * K + k], for tokens below vtc.
template <int PL, int TPW>
__device__ __forceinline__ void wave_topk(const float* __restrict__ scores, int64_t st,
                                          int64_t se, int E, int K, int vtc, int t0,
                                          int wave, int nwaves, int lane,
                                          int* __restrict__ sel) {
  constexpr int kTokPerWave = TPW;
  uint32_t ku[kTokPerWave][PL];
  int ke[kTokPerWave][PL];
  bool live[kTokPerWave];
  // loads first, all of them, from clamped (always valid) addresses; the
  // keys of dead tokens and of experts >= E are masked to 0 afterwards
  float sv[kTokPerWave][PL];
  // contiguous rows that every lane fills (E == 64 * PL) and 16-byte aligned
  // lane runs: one 16-byte load per 4 experts instead of four 4-byte loads
  const bool vec = (PL % 4 == 0) && se == 1 && E == kWave * PL && st % 4 == 0 &&
                   (reinterpret_cast<uintptr_t>(scores) & 15) == 0;
#pragma unroll
  for (int q = 0; q < kTokPerWave; ++q) {
    const int t = t0 + wave + q * nwaves;
    live[q] = t < vtc;  // wave-uniform
    const float* srow = scores + static_cast<int64_t>(live[q] ? t : 0) * st;
    if (vec) {
#pragma unroll
      for (int j = 0; j < PL; j += 4) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 v4 = *reinterpret_cast<const f32x4*>(srow + lane * PL + j);
        sv[q][j] = v4.x;
        if constexpr (PL >= 4) {
          sv[q][j + 1] = v4.y;
          sv[q][j + 2] = v4.z;
          sv[q][j + 3] = v4.w;
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < PL; ++j) {
        const int e = min(lane * PL + j, E - 1);
        sv[q][j] = srow[static_cast<int64_t>(e) * se];
      }
    }
  }
#pragma unroll
  for (int q = 0; q < kTokPerWave; ++q) {
#pragma unroll
    for (int j = 0; j < PL; ++j) {
      const int e = lane * PL + j;
      ke[q][j] = e;
      ku[q][j] = (live[q] && e < E) ? score_key(sv[q][j]) : 0u;
    }
    // stable insertion sort, descending key (ties keep ascending id)
#pragma unroll
    for (int i = 1; i < PL; ++i) {
#pragma unroll
      for (int j = i; j > 0; --j) {
        const bool sw = ku[q][j] > ku[q][j - 1];
        const uint32_t a = ku[q][j], b = ku[q][j - 1];
        const int ea = ke[q][j], eb = ke[q][j - 1];
        ku[q][j - 1] = sw ? a : b;
        ku[q][j] = sw ? b : a;
        ke[q][j - 1] = sw ? ea : eb;
        ke[q][j] = sw ? eb : ea;
      }
    }
  }
  int mine[kTokPerWave];  // lane k keeps slot k's expert
  for (int k = 0; k < K; ++k) {
    uint32_t head[kTokPerWave], m[kTokPerWave];
#pragma unroll
    for (int q = 0; q < kTokPerWave; ++q) head[q] = ku[q][0];
    wave_max_keys<kTokPerWave>(head, m);
#pragma unroll
    for (int q = 0; q < kTokPerWave; ++q) {
      const uint64_t tied = __ballot(ku[q][0] == m[q]);
      const int w = __builtin_ctzll(tied);  // lowest lane among the ties
      const int e_win = __builtin_amdgcn_readlane(ke[q][0], w);
      const bool pop = lane == w;
#pragma unroll
      for (int j = 0; j + 1 < PL; ++j) {
        ku[q][j] = pop ? ku[q][j + 1] : ku[q][j];
        ke[q][j] = pop ? ke[q][j + 1] : ke[q][j];
      }
      if (pop) ku[q][PL - 1] = 0u;
      mine[q] = lane == k ? e_win : mine[q];
    }
  }
#pragma unroll
  for (int q = 0; q < kTokPerWave; ++q)
    if (live[q] && lane < K) sel[(wave + q * nwaves) * K + lane] = mine[q];
}

// PL = expert candidates per lane (E <= 64 * PL); TPW = tokens per wave, so
// a block is 16 * TPW tokens (32, or 16 for small batches: one token per
// wave, half the top-k rounds on each wave's path).
template <int PL, int TPW>
__global__ __launch_bounds__(kSelThreads) void select_rank_kernel(
    const float* __restrict__ scores, int64_t st, int64_t se, int T, int E, int K,
    const int* __restrict__ vtc_ptr, int* __restrict__ pair, int* __restrict__ hist,
    int nblk) {
  __shared__ uint32_t mask[kMaxE];
  __shared__ int sel[kTokPerBlock * kMaxK];

  constexpr int kTpb = TPW * (kSelThreads / kWave);
  static_assert(kTpb <= kTokPerBlock, "one bit per token in a 32-bit mask");
  const int blk = blockIdx.x;
  const int t0 = blk * kTpb;
  const int vtc = clamp_count(vtc_ptr, T);
  const int lane = lane_id();
  const int wave = uniform(threadIdx.x >> 6);
  const int nwaves = kSelThreads / kWave;

  for (int e = threadIdx.x; e < E; e += kSelThreads) mask[e] = 0u;

  // ---- top-k: wave w owns tokens w and w+16 of the workgroup
  wave_topk<PL, TPW>(scores, st, se, E, K, vtc, t0, wave, nwaves, lane, sel);
  __syncthreads();

  // ---- one bit per valid token in each of its experts' masks
  const int npairs = kTpb * K;
  for (int p = threadIdx.x; p < npairs; p += kSelThreads) {
    const int tl = p / K;
    if (t0 + tl < vtc) atomicOr(&mask[sel[p]], 1u << tl);
  }
  __syncthreads();

  // ---- stable rank inside (block, expert) and the block histogram
  for (int p = threadIdx.x; p < npairs; p += kSelThreads) {
    const int tl = p / K;
    const int t = t0 + tl;
    if (t < vtc) {
      const int e = sel[p];
      const uint32_t before = mask[e] & ((1u << tl) - 1u);
      pair[static_cast<int64_t>(t0) * K + p] = e | (__popc(before) << 16);
    }
  }
  for (int e = threadIdx.x; e < E; e += kSelThreads)
    hist[static_cast<int64_t>(e) * nblk + blk] = __popc(mask[e]);
}

// Small batches, the whole shuffle in one launch: one workgroup takes the
// top-k of every token (TPW per wave, the fewest that cover T: up to 32 tokens
// with any E, up to 64 when the top-k rounds are short), ORs one bit per
// token into a 64-bit LDS mask per expert, and places every pair itself:
// expert e's rows start at the exclusive scan over experts of the mask
// popcounts, and a pair's rank is the popcount of the mask bits of the tokens
// before it.
constexpr int kSmallT = 64;
constexpr int kSmallWideE = 256;  // above this, up to 32 tokens
template <int PL, int TPW>
__global__ __launch_bounds__(kSelThreads) void shuffle_small_kernel(
    const float* __restrict__ scores, int64_t st, int64_t se, int T, int E, int K,
    const int* __restrict__ vtc_ptr, int* __restrict__ counts, int* __restrict__ ti,
    int* __restrict__ ei, int* __restrict__ rop) {
  __shared__ unsigned long long mask[kMaxE];
  __shared__ int sel[kSmallT * kMaxK];
  __shared__ int first[kMaxE];
  __shared__ int wave_tot[kSelThreads / kWave];
  // the workgroup has as many waves as hold the tokens, TPW each (at most 16)
  const int nt = blockDim.x;
  const int tid = threadIdx.x;
  const int vtc = clamp_count(vtc_ptr, T);
  const int lane = lane_id();
  const int wave = uniform(tid >> 6);
  const int nwaves = nt / kWave;

  for (int e = tid; e < E; e += nt) mask[e] = 0ull;
  static_assert(TPW * (kSelThreads / kWave) <= kSmallT, "tokens of one workgroup");
  wave_topk<PL, TPW>(scores, st, se, E, K, vtc, 0, wave, nwaves, lane, sel);
  __syncthreads();
  const int npairs = T * K;
  for (int p = tid; p < npairs; p += nt) {
    const int t = p / K;
    if (t < vtc) atomicOr(&mask[sel[p]], 1ull << t);
  }
  __syncthreads();

  // expert e's first row: thread i takes experts [i*per, i*per + per), their
  // counts summed, the sums scanned over the workgroup
  const int per = (E + nt - 1) / nt;
  const int e0 = tid * per;
  int mine = 0;
  for (int e = e0; e < min(e0 + per, E); ++e) mine += __popcll(mask[e]);
  int incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int base = incl - mine;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
  for (int e = e0; e < min(e0 + per, E); ++e) {
    const int c = __popcll(mask[e]);
    first[e] = base;
    counts[e] = c;
    base += c;
  }
  if (tid == 0) counts[E] = vtc * K;
  __syncthreads();

  for (int p = tid; p < npairs; p += nt) {
    const int t = p / K;
    if (t < vtc) {
      const int e = sel[p];
      const int r = first[e] + __popcll(mask[e] & ((1ull << t) - 1ull));
      ti[r] = t;
      ei[r] = e;
      if (rop) rop[p] = r;
    } else {
      ti[p] = t;
      ei[p] = -1;
      if (rop) rop[p] = -1;
    }
  }
}

// One wave per expert: exclusive scan of hist[e][0..nblk) in place (offsets
// of each block's pairs inside the expert's rows) and counts[e] = its total.
// Tiles of 256 blocks: lane l loads blocks 4l..4l+3 of the tile at once,
// scans them locally, and a wave scan of the lane sums adds the rest.
constexpr int kScanWaves = 4;
constexpr int kScanPer = 4;
__global__ __launch_bounds__(kScanWaves* kWave) void expert_scan_kernel(
    int* __restrict__ hist, int E, int nblk, int* __restrict__ counts) {
  const int lane = lane_id();
  const int e = blockIdx.x * kScanWaves + uniform(threadIdx.x >> 6);
  if (e >= E) return;
  int* row = hist + static_cast<int64_t>(e) * nblk;
  int carry = 0;
  for (int b0 = 0; b0 < nblk; b0 += kWave * kScanPer) {
    int v[kScanPer];
    int mine = 0;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      const int b = b0 + lane * kScanPer + i;
      v[i] = b < nblk ? row[b] : 0;
      mine += v[i];
    }
    int incl = mine;  // inclusive wave scan of the lane sums
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += o;
    }
    int run = carry + incl - mine;
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      const int b = b0 + lane * kScanPer + i;
      if (b < nblk) row[b] = run;
      run += v[i];
    }
    carry += __shfl(incl, kWave - 1, kWave);
  }
  if (lane == 0) counts[e] = carry;
}

constexpr int kPlaceThreads = 256;
__global__ __launch_bounds__(kPlaceThreads) void place_kernel(
    const int* __restrict__ pair, const int* __restrict__ offs, int nblk, int blk_shift, int T,
    int E, int K, const int* __restrict__ vtc_ptr, int* __restrict__ counts,
    int* __restrict__ ti, int* __restrict__ ei, int* __restrict__ rop) {
  __shared__ int first[kMaxE];
  __shared__ int wave_tot[kPlaceThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  // this thread's pair, loaded before the counts scan so the two overlap
  const int64_t p = static_cast<int64_t>(blockIdx.x) * kPlaceThreads + tid;
  const int64_t npairs = static_cast<int64_t>(T) * K;
  const bool have = p < npairs;
  const int t = have ? static_cast<int>(p / K) : 0;
  const int vtc = clamp_count(vtc_ptr, T);
  const int v = (have && t < vtc) ? pair[p] : 0;
  const int e = v & 0xFFFF;
  const int rank = v >> 16;
  const int off = (have && t < vtc) ? offs[static_cast<int64_t>(e) * nblk + (t >> blk_shift)] : 0;

  // first[e] = sum of counts[e'] for e' < e: each thread scans E/256 counts,
  // then waves and workgroup combine (E <= 1024 -> at most 4 per thread)
  constexpr int kPer = kMaxE / kPlaceThreads;
  int c[kPer];
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int ee = tid * kPer + i;
    c[i] = ee < E ? counts[ee] : 0;
    mine += c[i];
  }
  int incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int base = incl - mine;
  for (int w = 0; w < wave; ++w) base += wave_tot[w];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int ee = tid * kPer + i;
    if (ee < E) first[ee] = base;
    base += c[i];
  }
  __syncthreads();
  if (blockIdx.x == 0 && tid == 0) counts[E] = vtc * K;

  if (!have) return;
  if (t < vtc) {
    const int r = first[e] + off + rank;
    ti[r] = t;
    ei[r] = e;
    if (rop) rop[p] = r;
  } else {
    ti[p] = t;
    ei[p] = -1;
    if (rop) rop[p] = -1;
  }
}

// The expert scan and the placement in one launch, for histograms that fit
// in LDS (E * nblk <= kFuseHist ints). In expert-major order the exclusive
// scan of the flattened [E][nblk] histogram is, at (e, b), every row of the
// experts below e plus expert e's rows in blocks below b: exactly
// first[e] + offset[e][b]. Every workgroup runs that one scan (thread i owns
// entries 32i .. 32i+31: one local pass, a workgroup scan of the thread
// sums, the prefixes written to LDS with one pad word per 32 so the writes
// do not collide in a bank), then places its pairs. Workgroup 0 writes
// counts as differences of the prefixes at row starts.
constexpr int kFusePer = 32;
constexpr int kFuseHist = kPlaceThreads * kFusePer;  // 8192
__device__ __forceinline__ int fuse_pad(int i) { return i + (i >> 5); }

__global__ __launch_bounds__(kPlaceThreads) void scan_place_kernel(
    const int* __restrict__ pair, const int* __restrict__ hist, int nblk, int blk_shift, int T,
    int E, int K, const int* __restrict__ vtc_ptr, int* __restrict__ counts,
    int* __restrict__ ti, int* __restrict__ ei, int* __restrict__ rop) {
  __shared__ int pre[kFuseHist + kFuseHist / 32 + 1];
  __shared__ int wave_tot[kPlaceThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int64_t p = static_cast<int64_t>(blockIdx.x) * kPlaceThreads + tid;
  const int64_t npairs = static_cast<int64_t>(T) * K;
  const bool have = p < npairs;
  const int t = have ? static_cast<int>(p / K) : 0;
  const int vtc = clamp_count(vtc_ptr, T);
  const int v = (have && t < vtc) ? pair[p] : 0;
  const int e = v & 0xFFFF;
  const int rank = v >> 16;

  // this thread's entries, as 16-byte loads: hist is 256-byte aligned and
  // its workspace region is padded to 256 bytes, so a load that starts
  // below n stays inside it; entries >= n are taken as 0
  const int n = E * nblk;
  const int i0 = tid * kFusePer;
  int val[kFusePer];
  int mine = 0;
#pragma unroll
  for (int j = 0; j < kFusePer / 4; ++j) {
    const int i = i0 + 4 * j;
    const u32x4 q = i < n ? *reinterpret_cast<const u32x4*>(hist + i) : u32x4{0u, 0u, 0u, 0u};
    val[4 * j + 0] = i + 0 < n ? static_cast<int>(q.x) : 0;
    val[4 * j + 1] = i + 1 < n ? static_cast<int>(q.y) : 0;
    val[4 * j + 2] = i + 2 < n ? static_cast<int>(q.z) : 0;
    val[4 * j + 3] = i + 3 < n ? static_cast<int>(q.w) : 0;
  }
#pragma unroll
  for (int j = 0; j < kFusePer; ++j) mine += val[j];
  int incl = mine;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int run = incl - mine;
  int all = 0;
#pragma unroll
  for (int w = 0; w < kPlaceThreads / kWave; ++w) {
    run += w < wave ? wave_tot[w] : 0;
    all += wave_tot[w];
  }
#pragma unroll
  for (int j = 0; j < kFusePer; ++j) {
    if (i0 + j < n) pre[fuse_pad(i0 + j)] = run;
    run += val[j];
  }
  if (tid == 0) pre[fuse_pad(n)] = all;
  __syncthreads();

  if (blockIdx.x == 0) {
    for (int x = tid; x < E; x += kPlaceThreads)
      counts[x] = pre[fuse_pad((x + 1) * nblk)] - pre[fuse_pad(x * nblk)];
    if (tid == 0) counts[E] = vtc * K;
  }
  if (!have) return;
  if (t < vtc) {
    const int r = pre[fuse_pad(e * nblk + (t >> blk_shift))] + rank;
    ti[r] = t;
    ei[r] = e;
    if (rop) rop[p] = r;
  } else {
    ti[p] = t;
    ei[p] = -1;
    if (rop) rop[p] = -1;
  }
}

// counts[0..E] = 0 (no pairs at all)
__global__ void zero_counts_kernel(int* __restrict__ counts, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) counts[i] = 0;
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

}  // namespace

// Tokens per top-k block: 16 (one per wave) for batches of up to kHalfBlockT
// tokens, whose few blocks are latency-bound, else 32.
constexpr int kHalfBlockT = 128;
static int block_shift(int T) { return T <= kHalfBlockT ? 4 : 5; }

size_t shuffle_workspace_bytes(int T, int E, int K) {
  const int nblk = (T + (1 << block_shift(T)) - 1) >> block_shift(T);
  return align256(static_cast<size_t>(T) * K * sizeof(int)) +
         align256(static_cast<size_t>(E) * nblk * sizeof(int));
}

hipError_t launch_shuffle(const float* scores, int64_t st, int64_t se, int T, int E,
                          int K, const int* vtc, int* counts, int* expert_indices,
                          int* token_indices, int* row_of_pair, void* workspace,
                          hipStream_t stream) {
  if (T == 0) {
    hipLaunchKernelGGL(zero_counts_kernel, dim3((E + 1 + 255) / 256), dim3(256), 0, stream,
                       counts, E + 1);
    return hipGetLastError();
  }
  constexpr int kWaves = kSelThreads / kWave;
  // Up to 32 tokens a wave holds at most two, and one launch beats two (E =
  // 256, K = 8: 6.1 us at 32 tokens against 7.7 us for two launches at 64).
  // From 33 to 64 tokens a wave would hold four: the extra tokens' K rounds
  // (longer with more candidates per lane) outweigh the launch saved once
  // K * candidates per lane is above 8 (at 64 tokens: 9.3 us in one launch,
  // 7.7 us in two with 16-token blocks).
  const int pl_all = (E + kWave - 1) / kWave;
  if (T <= kSmallT / 2 || (T <= kSmallT && E <= kSmallWideE && K * pl_all <= 8)) {
    // one token per wave up to 16 tokens: as many waves as tokens
    const dim3 g(1), b(T <= kWaves ? T * kWave : kSelThreads);
#define MOE_SMALL(PLV, TPWV)                                                             \
  hipLaunchKernelGGL((shuffle_small_kernel<PLV, TPWV>), g, b, 0, stream, scores, st, se, T, \
                     E, K, vtc, counts, token_indices, expert_indices, row_of_pair)
    // the fewest tokens per wave that cover T: each wave's K top-k rounds run
    // for every token it holds, live or not
#define MOE_SMALL_T(PLV)                               \
  do {                                                 \
    if (T <= kWaves) MOE_SMALL(PLV, 1);                \
    else if (T <= 2 * kWaves) MOE_SMALL(PLV, 2);       \
    else MOE_SMALL(PLV, 4);                            \
  } while (0)
    const int pls = (E + kWave - 1) / kWave;
    if (E <= kSmallWideE) {
      if (pls <= 1) MOE_SMALL_T(1);
      else if (pls <= 2) MOE_SMALL_T(2);
      else MOE_SMALL_T(4);
    } else {
      // more than 256 experts: at most two tokens per wave (registers)
      if (pls <= 8) {
        if (T <= kWaves) MOE_SMALL(8, 1);
        else MOE_SMALL(8, 2);
      } else {
        if (T <= kWaves) MOE_SMALL(16, 1);
        else MOE_SMALL(16, 2);
      }
    }
#undef MOE_SMALL_T
#undef MOE_SMALL
    return hipGetLastError();
  }
  const int bs = block_shift(T);
  const int nblk = (T + (1 << bs) - 1) >> bs;
  char* ws = static_cast<char*>(workspace);
  int* pair = reinterpret_cast<int*>(ws);
  int* hist = reinterpret_cast<int*>(ws + align256(static_cast<size_t>(T) * K * sizeof(int)));
  const int pl = (E + kWave - 1) / kWave;
  const dim3 g1(nblk), b1(kSelThreads);
#define MOE_SEL2(PLV, TPWV)                                                                 \
  hipLaunchKernelGGL((select_rank_kernel<PLV, TPWV>), g1, b1, 0, stream, scores, st, se, T, \
                     E, K, vtc, pair, hist, nblk)
#define MOE_SEL(PLV)                       \
  do {                                     \
    if (bs == 4) MOE_SEL2(PLV, 1);         \
    else MOE_SEL2(PLV, 2);                 \
  } while (0)
  if (pl <= 1) MOE_SEL(1);
  else if (pl <= 2) MOE_SEL(2);
  else if (pl <= 4) MOE_SEL(4);
  else if (pl <= 8) MOE_SEL(8);
  else MOE_SEL(16);
#undef MOE_SEL
#undef MOE_SEL2
  const int64_t npairs = static_cast<int64_t>(T) * K;
  const int pblocks = static_cast<int>((npairs + kPlaceThreads - 1) / kPlaceThreads);
  if (static_cast<int64_t>(E) * nblk <= kFuseHist) {
    hipLaunchKernelGGL(scan_place_kernel, dim3(pblocks), dim3(kPlaceThreads), 0, stream, pair,
                       hist, nblk, bs, T, E, K, vtc, counts, token_indices, expert_indices,
                       row_of_pair);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(expert_scan_kernel, dim3((E + kScanWaves - 1) / kScanWaves),
                     dim3(kScanWaves * kWave), 0, stream, hist, E, nblk, counts);
  hipLaunchKernelGGL(place_kernel, dim3(pblocks), dim3(kPlaceThreads), 0, stream, pair, hist,
                     nblk, bs, T, E, K, vtc, counts, token_indices, expert_indices, row_of_pair);
  return hipGetLastError();
}

}  // namespace moe
