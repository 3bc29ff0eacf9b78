// Combine: add expert output rows back into token order, deterministically.
//
// [GS] "mslk/moe/gather_scatter.py", scatter_add_dense_tokens: each valid
// input row is added into out[token_indices[row]] (the pages use relaxed
// atomics, so their order of additions is not fixed). [LY] "mslk/moe/
// layers.py", _combine_outputs: out starts as the shared-expert output.
//
// Here each token is owned by one wave per row slice, which reads the token's
// initial row and its expert rows and writes the row once:
//   acc = f32(out[t]); acc += f32(in[r]) for its rows r in ascending order;
//   out[t] = bf16(acc).
// No atomics, one write per output element, and the same fp32 addition
// sequence on every run.
//
// Where a token's rows come from:
//  by_token  the inverse map row_of_pair[t, 0..K) written by the shuffle;
//            invalid slots dropped and the rest sorted in-wave. For top-1
//            and top-2 on more than 4096 (token, slice) waves a wave takes
//            four consecutive tokens' slice, their slots in one load.
//  general   only token_indices is known. Up to 1024 rows each wave finds
//            its token's rows itself, in ascending order, with no other
//            launch. Beyond that a CSR of rows per token is built first: up
//            to 4096 rows and tokens by one workgroup in LDS; up to 131072
//            rows in two launches (chunks of 1024 rows bucket their (row,
//            token) pairs by 128-token range, then one workgroup per range
//            counts its tokens' rows, scans and fills); beyond that in four
//            (count, scan, slot, fill). The order inside a token's list
//            depends on atomics, so the reduce kernel sorts each list
//            before adding.
//  padded    the general path over the static-shape expert-parallel layout
//            [EP, T_K, D]: each row is read from the slab of the rank that
//            owns its expert.
#include <limits.h>

#include "device.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kRowWaves = 4;
constexpr int kGroup = 4;  // rows in flight together in the general combine
constexpr int kMultiTok = 4;  // tokens per wave of the top-1/top-2 by-token combine
constexpr int kScanThreads = 1024;

__device__ __forceinline__ int clamp_count(const int* p, int hi) {
  if (!p) return hi;
  int v = *p;
  return v < 0 ? 0 : (v > hi ? hi : v);
}

// Ascending bitonic sort of one int per lane over aligned blocks of `width`
// lanes (a wave-uniform power of two, 1..64): lanes [0, width) end sorted.
// A token's rows sit in its first n <= width lanes, so only log2(width) of
// the six merge levels run (three for K = 8 instead of six: each level's
// lane exchanges are dependent LDS-pipe round trips).
__device__ __forceinline__ int wave_sort_asc(int v, int lane, int width) {
  for (int k = 2; k <= width; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int o = __shfl_xor(v, j, kWave);
      const bool up = (lane & k) == 0;
      const bool lower = (lane & j) == 0;
      v = (lower == up) ? min(v, o) : max(v, o);
    }
  }
  return v;
}

// The least power of two >= n, for 1 <= n <= 64.
__device__ __forceinline__ int sort_width(int n) {
  return n <= 1 ? 1 : 1 << (32 - __builtin_clz(static_cast<unsigned>(n - 1)));
}

// Loads group [i0, i0+G) of the n rows listed in ascending order in lanes
// 0..n-1 of sorted_rows. Every load is unconditional: positions past n re-read
// row n-1 (an L2 hit), so the G*CPL loads issue back to back with no branch
// or wait between them.
template <int CPL, int G, bool FULL>
__device__ __forceinline__ void load_rows(u32x4 (&buf)[G][CPL], const uint16_t* __restrict__ in,
                                          int D, int nch, int base, int sorted_rows, int i0,
                                          int n) {
#pragma unroll
  for (int q = 0; q < G; ++q) {
    const int r = __builtin_amdgcn_readlane(sorted_rows, min(i0 + q, n - 1));
    const uint16_t* src = in + static_cast<int64_t>(r) * D;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
      const int c = base + j * kWave;
      if (FULL || c < nch) buf[q][j] = ld16_stream(src + c * kChunk);
    }
  }
}

// acc += the group's rows that exist (positions i0+q < n), in order.
template <int CPL, int G, bool FULL>
__device__ __forceinline__ void add_group(float (&acc)[CPL][8], const u32x4 (&buf)[G][CPL],
                                          int nch, int base, int i0, int n) {
#pragma unroll
  for (int q = 0; q < G; ++q) {
    if (i0 + q < n) {
#pragma unroll
      for (int j = 0; j < CPL; ++j) {
        const int c = base + j * kWave;
        if (FULL || c < nch) {
          float f[8];
          unpack8(buf[q][j], f);
#pragma unroll
          for (int i = 0; i < 8; ++i) acc[j][i] = acc[j][i] + f[i];
        }
      }
    }
  }
}

// acc[j] (this lane's CPL chunks of the slice) += the n rows listed in
// ascending order in lanes 0..n-1 of `sorted_rows`.
template <int CPL, int G, bool FULL>
__device__ __forceinline__ void add_rows(float (&acc)[CPL][8], const uint16_t* __restrict__ in,
                                         int D, int nch, int base, int sorted_rows, int n) {
  for (int i0 = 0; i0 < n; i0 += G) {
    u32x4 buf[G][CPL];
    load_rows<CPL, G, FULL>(buf, in, D, nch, base, sorted_rows, i0, n);
    add_group<CPL, G, FULL>(acc, buf, nch, base, i0, n);
  }
}

template <int CPL, bool FULL>
__device__ __forceinline__ void load_acc(float (&acc)[CPL][8], const uint16_t* __restrict__ row,
                                         int nch, int base) {
  u32x4 v[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = base + j * kWave;
    v[j] = (FULL || c < nch) ? ld16(row + c * kChunk) : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < CPL; ++j) unpack8(v[j], acc[j]);
}

// Packs every chunk before the first store, so that no store's data
// registers are reused while it is in flight.
template <int CPL, bool FULL>
__device__ __forceinline__ void store_acc(const float (&acc)[CPL][8], uint16_t* __restrict__ row,
                                          int nch, int base) {
  u32x4 o[CPL];
#pragma unroll
  for (int j = 0; j < CPL; ++j) o[j] = pack8(acc[j]);
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = base + j * kWave;
    if (FULL || c < nch) st16_stream(row + c * kChunk, o[j]);
  }
}

// This lane's chunks of the initial (output) row.
template <int CPL, bool FULL>
__device__ __forceinline__ void load_init(u32x4 (&o0)[CPL], const uint16_t* __restrict__ orow,
                                          int nch, int base) {
#pragma unroll
  for (int j = 0; j < CPL; ++j) {
    const int c = base + j * kWave;
    o0[j] = (FULL || c < nch) ? ld16(orow + c * kChunk) : u32x4{0u, 0u, 0u, 0u};
  }
}

// The per-token reduction of one slice from its loaded initial row o0: the
// first G expert rows are loaded, then added in order; later groups follow;
// one store. n >= 1.
template <int CPL, int G, bool FULL>
__device__ __forceinline__ void reduce_slice_from(const u32x4 (&o0)[CPL],
                                                  uint16_t* __restrict__ orow,
                                                  const uint16_t* __restrict__ in, int D,
                                                  int nch, int base, int sorted_rows, int n) {
  u32x4 buf[G][CPL];
  load_rows<CPL, G, FULL>(buf, in, D, nch, base, sorted_rows, 0, n);
  float acc[CPL][8];
#pragma unroll
  for (int j = 0; j < CPL; ++j) unpack8(o0[j], acc[j]);
  add_group<CPL, G, FULL>(acc, buf, nch, base, 0, n);
  for (int i0 = G; i0 < n; i0 += G) {
    load_rows<CPL, G, FULL>(buf, in, D, nch, base, sorted_rows, i0, n);
    add_group<CPL, G, FULL>(acc, buf, nch, base, i0, n);
  }
  store_acc<CPL, FULL>(acc, orow, nch, base);
}

// One (token, slice) of the by-token combine. The initial row does not depend
// on the slot rows: when the token is likely routed (t * K < V, true for
// every token below a shuffle's valid count) it is loaded before them, so the
// two loads overlap instead of following one another.
template <int CPL, int G, bool FULL>
__device__ __forceinline__ void scatter_token(uint16_t* __restrict__ out,
                                              const uint16_t* __restrict__ in,
                                              const int* __restrict__ rop, int t, int K, int V,
                                              int D, int nch, int base, int lane) {
  int r = lane < K ? rop[static_cast<int64_t>(t) * K + lane] : -1;
  uint16_t* orow = out + static_cast<int64_t>(t) * D;
  const bool early = static_cast<int64_t>(t) * K < V;  // wave-uniform
  u32x4 o0[CPL];
  if (early) load_init<CPL, FULL>(o0, orow, nch, base);
  const bool ok = r >= 0 && r < V;
  const int n = __popcll(__ballot(ok));
  if (n == 0) return;
  // slots sit in lanes [0, K): sorting K lanes (rounded up) is enough
  const int sorted_rows = wave_sort_asc(ok ? r : INT_MAX, lane, sort_width(uniform(K)));
  if (!early) load_init<CPL, FULL>(o0, orow, nch, base);
  reduce_slice_from<CPL, G, FULL>(o0, orow, in, D, nch, base, sorted_rows, n);
}

template <int CPL, int G>
__global__ __launch_bounds__(kRowWaves* kWave) void scatter_tokens_kernel(
    uint16_t* __restrict__ out, int T, const uint16_t* __restrict__ in,
    const int* __restrict__ rop, int K, int a, int D, const int* __restrict__ vrows,
    int nsl) {
  const int lane = lane_id();
  const int64_t unit =
      static_cast<int64_t>(blockIdx.x) * kRowWaves + uniform(threadIdx.x >> 6);
  const int t = static_cast<int>(unit / nsl);
  const int sl = static_cast<int>(unit - static_cast<int64_t>(t) * nsl);
  if (t >= T) return;
  const int V = clamp_count(vrows, a);
  const int nch = D >> 3;
  const int slice0 = sl * kWave * CPL;
  if (slice0 + kWave * CPL <= nch)
    scatter_token<CPL, G, true>(out, in, rop, t, K, V, D, nch, slice0 + lane, lane);
  else
    scatter_token<CPL, G, false>(out, in, rop, t, K, V, D, nch, slice0 + lane, lane);
}

// M consecutive tokens' same slice in one wave, for top-k of at most KP (1 or
// 2) slots: lanes m*KP .. m*KP+KP-1 load token m's slots in one coalesced
// load, each token's lanes are put in ascending row order, and the M initial rows
// and all the tokens' rows are in flight together before the first add. The
// index round trip is paid once per M slices instead of once per slice. The
// additions are those of scatter_token, in the same order.
template <int CPL, int M, int KP, bool FULL>
__device__ __forceinline__ void scatter_tokens_m(uint16_t* __restrict__ out,
                                                 const uint16_t* __restrict__ in,
                                                 const int* __restrict__ rop, int t0, int T,
                                                 int K, int V, int D, int nch, int base,
                                                 int lane) {
  static_assert(M * KP <= kWave && (KP == 1 || KP == 2), "one slot per lane");
  const int m_l = lane / KP;
  const int s_l = lane % KP;
  const int t_l = t0 + m_l;
  const int r = (m_l < M && s_l < K && t_l < T) ? rop[static_cast<int64_t>(t_l) * K + s_l] : -1;
  u32x4 o0[M][CPL];
  bool early[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int tm = t0 + m;
    early[m] = tm < T && static_cast<int64_t>(tm) * K < V;  // wave-uniform
    if (early[m]) load_init<CPL, FULL>(o0[m], out + static_cast<int64_t>(tm) * D, nch, base);
  }
  const bool ok = r >= 0 && r < V;
  const uint64_t okm = __ballot(ok);
  // each token's KP lanes ascending, invalid slots (INT_MAX) last; for KP = 2
  // one compare-exchange per lane pair (wave_sort_asc orders only its first
  // block ascending: its last stage alternates direction from block to block)
  int sorted = ok ? r : INT_MAX;
  if constexpr (KP == 2) {
    const int o = __shfl_xor(sorted, 1, kWave);
    sorted = (lane & 1) ? max(sorted, o) : min(sorted, o);
  }
  int n[M];
  u32x4 buf[M][KP][CPL];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    n[m] = __popcll((okm >> (m * KP)) & ((1ull << KP) - 1ull));
    if (n[m] > 0) {
#pragma unroll
      for (int q = 0; q < KP; ++q) {
        const int row = __builtin_amdgcn_readlane(sorted, m * KP + min(q, n[m] - 1));
        const uint16_t* src = in + static_cast<int64_t>(row) * D;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const int c = base + j * kWave;
          if (FULL || c < nch) buf[m][q][j] = ld16_stream(src + c * kChunk);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m)
    if (n[m] > 0 && !early[m])
      load_init<CPL, FULL>(o0[m], out + static_cast<int64_t>(t0 + m) * D, nch, base);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    if (n[m] == 0) continue;
    float acc[CPL][8];
#pragma unroll
    for (int j = 0; j < CPL; ++j) unpack8(o0[m][j], acc[j]);
#pragma unroll
    for (int q = 0; q < KP; ++q) {
      if (q < n[m]) {
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
          const int c = base + j * kWave;
          if (FULL || c < nch) {
            float f[8];
            unpack8(buf[m][q][j], f);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[j][i] = acc[j][i] + f[i];
          }
        }
      }
    }
    store_acc<CPL, FULL>(acc, out + static_cast<int64_t>(t0 + m) * D, nch, base);
  }
}

template <int CPL, int M, int KP>
__global__ __launch_bounds__(kRowWaves* kWave) void scatter_tokens_multi_kernel(
    uint16_t* __restrict__ out, int T, const uint16_t* __restrict__ in,
    const int* __restrict__ rop, int K, int a, int D, const int* __restrict__ vrows,
    int nsl) {
  const int lane = lane_id();
  const int64_t unit =
      static_cast<int64_t>(blockIdx.x) * kRowWaves + uniform(threadIdx.x >> 6);
  const int g = static_cast<int>(unit / nsl);
  const int sl = static_cast<int>(unit - static_cast<int64_t>(g) * nsl);
  const int64_t t0 = static_cast<int64_t>(g) * M;
  if (t0 >= T) return;
  const int V = clamp_count(vrows, a);
  const int nch = D >> 3;
  const int slice0 = sl * kWave * CPL;
  if (slice0 + kWave * CPL <= nch)
    scatter_tokens_m<CPL, M, KP, true>(out, in, rop, static_cast<int>(t0), T, K, V, D, nch,
                                       slice0 + lane, lane);
  else
    scatter_tokens_m<CPL, M, KP, false>(out, in, rop, static_cast<int>(t0), T, K, V, D, nch,
                                        slice0 + lane, lane);
}

// ---------------------------------------------------------------- general
__global__ void csr_zero_kernel(int* __restrict__ cnt, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) cnt[i] = 0;
}

// Rows whose token index is out of [0, T) are skipped (no fault).
__global__ void csr_count_kernel(const int* __restrict__ ti, int T, int a,
                                 const int* __restrict__ vrows, int* __restrict__ cnt,
                                 int* __restrict__ slot) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  const int V = clamp_count(vrows, a);
  if (r >= V) return;
  const int t = ti[r];
  if (static_cast<unsigned>(t) < static_cast<unsigned>(T)) slot[r] = atomicAdd(&cnt[t], 1);
}

// Exclusive scan of cnt[0..n) in place (one workgroup); cnt[n] = total.
// Tiles of kScanThreads * kScanPer counts: one coalesced load of the whole
// tile, a transpose through LDS so each thread owns kScanPer consecutive
// counts, a workgroup scan of the per-thread sums, and one coalesced store.
constexpr int kScanPer = 8;
__global__ __launch_bounds__(kScanThreads) void csr_scan_kernel(int* __restrict__ cnt, int n) {
  __shared__ int tile[kScanThreads * kScanPer];
  __shared__ int wave_tot[kScanThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  constexpr int kTile = kScanThreads * kScanPer;
  int carry = 0;
  for (int base = 0; base < n; base += kTile) {
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      const int i = base + k * kScanThreads + tid;
      tile[k * kScanThreads + tid] = i < n ? cnt[i] : 0;
    }
    __syncthreads();
    int v[kScanPer];
    int mine = 0;
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      v[k] = tile[tid * kScanPer + k];
      mine += v[k];
    }
    int incl = mine;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int o = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    int run = carry + incl - mine;
    int tile_total = 0;
    for (int w = 0; w < kScanThreads / kWave; ++w) {
      const int wt = wave_tot[w];
      if (w < wave) run += wt;
      tile_total += wt;
    }
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      tile[tid * kScanPer + k] = run;
      run += v[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kScanPer; ++k) {
      const int i = base + k * kScanThreads + tid;
      if (i < n) cnt[i] = tile[k * kScanThreads + tid];
    }
    carry += tile_total;
    __syncthreads();  // tile and wave_tot are reused by the next tile
  }
  if (tid == 0) cnt[n] = carry;
}

__global__ void csr_fill_kernel(const int* __restrict__ ti, int T, int a,
                                const int* __restrict__ vrows, const int* __restrict__ start,
                                const int* __restrict__ slot, int* __restrict__ list) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  const int V = clamp_count(vrows, a);
  if (r >= V) return;
  const int t = ti[r];
  if (static_cast<unsigned>(t) < static_cast<unsigned>(T)) list[start[t] + slot[r]] = r;
}

// The CSR in two launches, for up to kRangeMaxRows rows and kMaxRanges
// token ranges of kRangeT tokens:
//  csr_bucket  one workgroup per kBucketRows rows (one per thread): groups its
//              rows by token range in LDS (counting sort over the ranges) and
//              writes them range by range as (row, token) pairs, with each
//              range's count and chunk-local start ([range][chunk] matrices).
//  csr_range   one workgroup per token range: finds its rows in every chunk
//              from the two matrices (its place in the final list is the sum
//              of its chunk-local starts), counts them per token in LDS --
//              each row taking its slot within its token and staged in LDS --
//              scans the counts into start[], and writes each staged row to
//              start + slot.
// Each workgroup reads only its own rows. With counts (the padded layout)
// every bucket workgroup takes the valid row count from the expert prefix,
// which workgroup 0 also writes (prefix[0..E], prefix[E] = rows covered,
// clamped to a). The order inside a token's list follows the LDS atomics; the
// reduce kernels sort it.
constexpr int kRangeT = 128;           // tokens per range
constexpr int kRangeMaxRows = 131072;  // rows the two-launch build takes
constexpr int kBucketRows = kScanThreads;
constexpr int kMaxChunks = kRangeMaxRows / kBucketRows;  // 128
constexpr int kMaxRanges = 2048;
constexpr int kRangeStage = 8192;      // a range's rows kept in LDS for the fill
static_assert(kRangeT <= 256, "the staged fill packs the token offset in 8 bits");
static_assert(kMaxRanges <= 2 * kScanThreads, "the bucket scan takes two ranges per thread");

// Exclusive scan of one value per thread over a workgroup of NT threads;
// `total` gets the sum. Syncs the workgroup; wave_tot holds NT / 64 entries.
template <int NT = kScanThreads>
__device__ __forceinline__ int block_excl_scan(int v, int lane, int wave, int* wave_tot,
                                               int& total) {
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NT / kWave; ++w) {
    const int wt = wave_tot[w];
    if (w < wave) base += wt;
    total += wt;
  }
  return base + incl - v;
}

// The valid row count: min(sum of counts, a) with counts (workgroup 0 writes
// the expert prefix), else *vrows clamped to [0, a]. Syncs the workgroup.
__device__ __forceinline__ int csr_valid_rows(const int* __restrict__ vrows,
                                              const int* __restrict__ counts, int E, int a,
                                              int* __restrict__ prefix, int lane, int wave,
                                              int* wave_tot) {
  if (!counts) return clamp_count(vrows, a);
  const int tid = threadIdx.x;
  const int v = tid < E ? max(counts[tid], 0) : 0;  // E <= kScanThreads
  int total;
  const int excl = block_excl_scan(v, lane, wave, wave_tot, total);
  if (blockIdx.x == 0) {
    if (tid < E) prefix[tid] = min(excl, a);
    if (tid == 0) prefix[E] = min(total, a);
  }
  return min(total, a);
}

__global__ __launch_bounds__(kScanThreads) void csr_bucket_kernel(
    const int* __restrict__ ti, int T, int a, const int* __restrict__ vrows,
    const int* __restrict__ counts, int E, int* __restrict__ prefix, int nrange, int G,
    int* __restrict__ rcnt, int* __restrict__ roff, int2* __restrict__ packed) {
  __shared__ int hist[kMaxRanges];
  __shared__ int wave_tot[2][kScanThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int g = blockIdx.x;
  const int r = g * kBucketRows + tid;
  const int t_raw = r < a ? ti[r] : -1;  // issued before the valid count is known
  for (int i = tid; i < nrange; i += kScanThreads) hist[i] = 0;
  const int V = csr_valid_rows(vrows, counts, E, a, prefix, lane, wave, wave_tot[0]);
  const int t = r < V ? t_raw : -1;
  const bool valid = static_cast<unsigned>(t) < static_cast<unsigned>(T);
  const int q = valid ? t / kRangeT : 0;
  __syncthreads();
  const int pos = valid ? atomicAdd(&hist[q], 1) : 0;
  __syncthreads();
  // chunk-local starts of the ranges: two ranges per thread
  const int c0 = 2 * tid < nrange ? hist[2 * tid] : 0;
  const int c1 = 2 * tid + 1 < nrange ? hist[2 * tid + 1] : 0;
  int total;
  const int s0 = block_excl_scan(c0 + c1, lane, wave, wave_tot[1], total);
  if (2 * tid < nrange) {
    rcnt[static_cast<int64_t>(2 * tid) * G + g] = c0;
    roff[static_cast<int64_t>(2 * tid) * G + g] = s0;
  }
  if (2 * tid + 1 < nrange) {
    rcnt[static_cast<int64_t>(2 * tid + 1) * G + g] = c1;
    roff[static_cast<int64_t>(2 * tid + 1) * G + g] = s0 + c0;
  }
  __syncthreads();  // every count read before the starts overwrite them
  if (2 * tid < nrange) hist[2 * tid] = s0;
  if (2 * tid + 1 < nrange) hist[2 * tid + 1] = s0 + c0;
  __syncthreads();
  if (valid) packed[static_cast<int64_t>(g) * kBucketRows + hist[q] + pos] = make_int2(r, t);
}

constexpr int kRangeThreads = 1024;  // at least one thread per token of a range
static_assert(kRangeThreads >= kRangeT && kMaxChunks <= kRangeThreads, "range kernel shape");
__global__ __launch_bounds__(kRangeThreads) void csr_range_kernel(
    int T, int G, const int* __restrict__ rcnt, const int* __restrict__ roff,
    const int2* __restrict__ packed, int* __restrict__ start, int* __restrict__ list) {
  __shared__ int cnt[kRangeT];
  __shared__ int seg[kMaxChunks + 1];  // exclusive prefix of this range's chunk counts
  __shared__ int soff[kMaxChunks];     // chunk-local start of this range
  __shared__ int wave_tot[3][kRangeThreads / kWave];
  __shared__ int stage_row[kRangeStage];
  __shared__ int stage_pos[kRangeStage];  // token offset | slot << 8
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int q = blockIdx.x;
  const int lo = q * kRangeT;
  const int n = min(kRangeT, T - lo);
  const int c = tid < G ? rcnt[static_cast<int64_t>(q) * G + tid] : 0;
  const int o = tid < G ? roff[static_cast<int64_t>(q) * G + tid] : 0;
  if (tid < kRangeT) cnt[tid] = 0;
  int nq;
  const int sc = block_excl_scan<kRangeThreads>(c, lane, wave, wave_tot[0], nq);  // syncs
  int base;
  (void)block_excl_scan<kRangeThreads>(o, lane, wave, wave_tot[1], base);         // rows of lower ranges
  if (tid < G) {
    seg[tid] = sc;
    soff[tid] = o;
  }
  if (tid == 0) seg[G] = nq;
  __syncthreads();

  // count: row i of the range sits in chunk g with seg[g] <= i < seg[g+1]
  const bool staged = nq <= kRangeStage;
  for (int i = tid; i < nq; i += kRangeThreads) {
    int lo_g = 0, hi_g = G;  // seg[lo_g] <= i < seg[hi_g]
    while (hi_g - lo_g > 1) {
      const int mid = (lo_g + hi_g) >> 1;
      if (seg[mid] <= i) lo_g = mid;
      else hi_g = mid;
    }
    const int2 e = packed[static_cast<int64_t>(lo_g) * kBucketRows + soff[lo_g] + (i - seg[lo_g])];
    const int rel = e.y - lo;
    const int slot = atomicAdd(&cnt[rel], 1);
    if (staged) {
      stage_row[i] = e.x;
      stage_pos[i] = rel | (slot << 8);
    }
  }
  __syncthreads();

  // exclusive scan of the range's counters (one per thread), offset by base
  const int cv = tid < n ? cnt[tid] : 0;
  int range_total;
  const int pos = base + block_excl_scan<kRangeThreads>(cv, lane, wave, wave_tot[2], range_total);
  if (tid < n) {
    start[lo + tid] = pos;
    cnt[tid] = pos;
  }
  if (lo + n == T && tid == 0) start[T] = base + range_total;
  __syncthreads();

  if (staged) {
    for (int i = tid; i < nq; i += kRangeThreads) {
      const int p = stage_pos[i];
      list[cnt[p & 0xFF] + (p >> 8)] = stage_row[i];
    }
    return;
  }
  // more rows than the stage holds: read them again, each row taking the next
  // free position of its token
  for (int i = tid; i < nq; i += kRangeThreads) {
    int lo_g = 0, hi_g = G;
    while (hi_g - lo_g > 1) {
      const int mid = (lo_g + hi_g) >> 1;
      if (seg[mid] <= i) lo_g = mid;
      else hi_g = mid;
    }
    const int2 e = packed[static_cast<int64_t>(lo_g) * kBucketRows + soff[lo_g] + (i - seg[lo_g])];
    list[atomicAdd(&cnt[e.y - lo], 1)] = e.x;
  }
}

// Small builds (up to kSmallRows rows and kSmallTok tokens) in one
// workgroup and one launch: each valid row's token and its slot within the
// token (an LDS atomic on the token's counter) stay in LDS, the counters are
// scanned into start[], and each row goes to start[t] + slot. The order inside
// a token's list depends on the atomics, as in the larger builds.
constexpr int kSmallRows = 4096;
constexpr int kSmallTok = 4096;
static_assert(kSmallTok % kScanThreads == 0, "the token scan takes whole runs per thread");
__global__ __launch_bounds__(kScanThreads) void csr_small_kernel(
    const int* __restrict__ ti, int T, int a, const int* __restrict__ vrows,
    const int* __restrict__ counts, int E, int* __restrict__ prefix, int* __restrict__ start,
    int* __restrict__ list) {
  __shared__ int cnt[kSmallTok];
  __shared__ int tok[kSmallRows];
  __shared__ int slot[kSmallRows];
  __shared__ int wave_tot[2][kScanThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  for (int i = tid; i < T; i += kScanThreads) cnt[i] = 0;
  const int V = csr_valid_rows(vrows, counts, E, a, prefix, lane, wave, wave_tot[0]);
  __syncthreads();
  for (int r = tid; r < V; r += kScanThreads) {
    const int t = ti[r];
    const bool valid = static_cast<unsigned>(t) < static_cast<unsigned>(T);
    tok[r] = valid ? t : -1;
    if (valid) slot[r] = atomicAdd(&cnt[t], 1);
  }
  __syncthreads();
  // exclusive scan of the counters: thread i owns tokens [i*kPer, i*kPer + kPer)
  constexpr int kPer = kSmallTok / kScanThreads;
  int c[kPer];
  int mine = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = tid * kPer + q;
    c[q] = i < T ? cnt[i] : 0;
    mine += c[q];
  }
  int total;
  int ex = block_excl_scan(mine, lane, wave, wave_tot[1], total);  // syncs
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int i = tid * kPer + q;
    if (i < T) {
      start[i] = ex;
      cnt[i] = ex;
    }
    ex += c[q];
  }
  if (tid == 0) start[T] = total;
  __syncthreads();
  for (int r = tid; r < V; r += kScanThreads) {
    const int t = tok[r];
    if (t >= 0) list[cnt[t] + slot[r]] = r;
  }
}

// Small general combines (up to kScanRows rows): each (token, slice) wave
// finds its token's rows itself, with no row-list build and so no launch
// before it. The wave loads all the token indices at once and adds the rows
// it finds in ascending order, in batches of up to 64, kScanG in flight.
constexpr int kScanRows = 1024;
constexpr int kScanChunks = kScanRows / kWave;
constexpr int kScanG = 8;
template <int CPL, bool FULL>
__device__ __forceinline__ void scan_reduce(uint16_t* __restrict__ orow,
                                            const uint16_t* __restrict__ in,
                                            const int (&tv)[kScanChunks], int V, int t, int D,
                                            int nch, int base, int lane, int* stage) {
  float acc[CPL][8];
  load_acc<CPL, FULL>(acc, orow, nch, base);
  const int n = for_token_rows(tv, V, t, lane, stage, [&](int rows, int nb) {
    add_rows<CPL, kScanG, FULL>(acc, in, D, nch, base, rows, nb);
  });
  if (n) store_acc<CPL, FULL>(acc, orow, nch, base);
}

template <int CPL>
__global__ __launch_bounds__(kRowWaves* kWave) void scatter_scan_kernel(
    uint16_t* __restrict__ out, int T, const uint16_t* __restrict__ in,
    const int* __restrict__ ti, int a, int D, const int* __restrict__ vrows, int nsl) {
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
  const int slice0 = sl * kWave * CPL;
  uint16_t* orow = out + static_cast<int64_t>(t) * D;
  if (slice0 + kWave * CPL <= nch)
    scan_reduce<CPL, true>(orow, in, tv, V, t, D, nch, slice0 + lane, lane, stage[wv]);
  else
    scan_reduce<CPL, false>(orow, in, tv, V, t, D, nch, slice0 + lane, lane, stage[wv]);
}

template <int CPL>
__global__ __launch_bounds__(kRowWaves* kWave) void scatter_csr_kernel(
    uint16_t* __restrict__ out, int T, const uint16_t* __restrict__ in,
    const int* __restrict__ start, const int* __restrict__ list, int D, int nsl) {
  const int lane = lane_id();
  const int64_t unit =
      static_cast<int64_t>(blockIdx.x) * kRowWaves + uniform(threadIdx.x >> 6);
  const int t = static_cast<int>(unit / nsl);
  const int sl = static_cast<int>(unit - static_cast<int64_t>(t) * nsl);
  if (t >= T) return;
  const int beg = start[t];
  const int n = start[t + 1] - beg;
  if (n == 0) return;

  const int nch = D >> 3;
  const int slice0 = sl * kWave * CPL;
  const int base = slice0 + lane;
  uint16_t* orow = out + static_cast<int64_t>(t) * D;
  if (n <= kWave) {
    // the initial row does not depend on the row list: load it alongside
    const bool full = slice0 + kWave * CPL <= nch;
    u32x4 o0[CPL];
    if (full)
      load_init<CPL, true>(o0, orow, nch, base);
    else
      load_init<CPL, false>(o0, orow, nch, base);
    const int r = lane < n ? list[beg + lane] : INT_MAX;
    const int sorted_rows = wave_sort_asc(r, lane, sort_width(uniform(n)));
    if (full)
      reduce_slice_from<CPL, kGroup, true>(o0, orow, in, D, nch, base, sorted_rows, n);
    else
      reduce_slice_from<CPL, kGroup, false>(o0, orow, in, D, nch, base, sorted_rows, n);
  } else {
    float acc[CPL][8];
    load_acc<CPL, false>(acc, orow, nch, base);
    // long list: take the rows in ascending order one at a time (each step a
    // wave-wide minimum over the rows above the previous one)
    int prev = -1;
    for (int i = 0; i < n; ++i) {
      int m = INT_MAX;
      for (int q = lane; q < n; q += kWave) {
        const int r = list[beg + q];
        if (r > prev && r < m) m = r;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = min(m, __shfl_xor(m, off, kWave));
      prev = m;
      add_rows<CPL, 1, false>(acc, in, D, nch, base, m, 1);
    }
    store_acc<CPL, false>(acc, orow, nch, base);
  }
}

// ---------------------------------------------------------------- padded
// [GS] scatter_add_padded_tokens: rows [off_e, off_e + counts[e]) of the
// shuffle's order belong to expert e and are read from rank e / (E / EP)'s
// slab of in [EP, T_K, D] at the same row positions.
constexpr int kMaxPaddedE = 1024;

// prefix[e] = sum of counts[e'] for e' < e (e <= E); prefix[E] is clamped to
// T_K and is the valid row count V of the CSR build. One workgroup.
__global__ __launch_bounds__(kScanThreads) void padded_prefix_kernel(
    const int* __restrict__ counts, int E, int T_K, int* __restrict__ prefix) {
  __shared__ int wave_tot[kScanThreads / kWave];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid >> 6;
  const int v = tid < E ? max(counts[tid], 0) : 0;  // E <= kScanThreads
  int incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += u;
  }
  if (lane == kWave - 1) wave_tot[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < kScanThreads / kWave; ++w) {
    if (w < wave) base += wave_tot[w];
    total += wave_tot[w];
  }
  if (tid < E) prefix[tid] = min(base + incl - v, T_K);
  if (tid == 0) prefix[E] = min(total, T_K);
}

// Rank owning row r: the expert e with prefix[e] <= r < prefix[e+1], over E/EP.
__device__ __forceinline__ int rank_of_row(const int* __restrict__ pre, int E, int epr, int r) {
  int lo = 0, hi = E;  // invariant: pre[lo] <= r < pre[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid] <= r) lo = mid;
    else hi = mid;
  }
  return lo / epr;
}

template <int CPL>
__global__ __launch_bounds__(kRowWaves* kWave) void scatter_padded_kernel(
    uint16_t* __restrict__ out, int T, const uint16_t* __restrict__ in, int T_K, int E, int EP,
    const int* __restrict__ prefix, const int* __restrict__ start, const int* __restrict__ list,
    int D, int nsl) {
  __shared__ int pre[kMaxPaddedE + 1];
  for (int e = threadIdx.x; e <= E; e += blockDim.x) pre[e] = prefix[e];
  __syncthreads();
  const int lane = lane_id();
  const int64_t unit =
      static_cast<int64_t>(blockIdx.x) * kRowWaves + uniform(threadIdx.x >> 6);
  const int t = static_cast<int>(unit / nsl);
  const int sl = static_cast<int>(unit - static_cast<int64_t>(t) * nsl);
  if (t >= T) return;
  const int beg = start[t];
  const int n = start[t + 1] - beg;
  if (n == 0) return;
  const int epr = E / EP;
  const int nch = D >> 3;
  const int slice0 = sl * kWave * CPL;
  const int base = slice0 + lane;
  uint16_t* orow = out + static_cast<int64_t>(t) * D;
  if (n <= kWave) {
    // the initial row does not depend on the row list: load it alongside
    const bool full = slice0 + kWave * CPL <= nch;
    u32x4 o0[CPL];
    if (full)
      load_init<CPL, true>(o0, orow, nch, base);
    else
      load_init<CPL, false>(o0, orow, nch, base);
    const int r = lane < n ? list[beg + lane] : INT_MAX;
    const int sorted = wave_sort_asc(r, lane, sort_width(uniform(n)));
    // source row of each sorted row: rank * T_K + row (ascending row order kept)
    const int src = lane < n ? rank_of_row(pre, E, epr, sorted) * T_K + sorted : 0;
    if (full)
      reduce_slice_from<CPL, kGroup, true>(o0, orow, in, D, nch, base, src, n);
    else
      reduce_slice_from<CPL, kGroup, false>(o0, orow, in, D, nch, base, src, n);
  } else {
    float acc[CPL][8];
    load_acc<CPL, false>(acc, orow, nch, base);
    int prev = -1;
    for (int i = 0; i < n; ++i) {
      int m = INT_MAX;
      for (int q = lane; q < n; q += kWave) {
        const int r = list[beg + q];
        if (r > prev && r < m) m = r;
      }
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) m = min(m, __shfl_xor(m, off, kWave));
      prev = m;
      add_rows<CPL, 1, false>(acc, in, D, nch, base, rank_of_row(pre, E, epr, m) * T_K + m, 1);
    }
    store_acc<CPL, false>(acc, orow, nch, base);
  }
}

// Small padded combines (T_K <= kScanRows): no row-list build. Each
// workgroup scans the expert counts into an LDS prefix; each (token, slice)
// wave then finds its token's rows among the first V = prefix[E] as the
// general scan combine does, and reads each from its owner rank's slab.
template <int CPL, bool FULL>
__device__ __forceinline__ void padded_scan_reduce(uint16_t* __restrict__ orow,
                                                   const uint16_t* __restrict__ in, int T_K,
                                                   const int* pre, int E, int epr,
                                                   const int (&tv)[kScanChunks], int V, int t,
                                                   int D, int nch, int base, int lane,
                                                   int* stage) {
  float acc[CPL][8];
  load_acc<CPL, FULL>(acc, orow, nch, base);
  const int n = for_token_rows(tv, V, t, lane, stage, [&](int rows, int nb) {
    const int src = lane < nb ? rank_of_row(pre, E, epr, rows) * T_K + rows : 0;
    add_rows<CPL, kScanG, FULL>(acc, in, D, nch, base, src, nb);
  });
  if (n) store_acc<CPL, FULL>(acc, orow, nch, base);
}

// The expert prefix of the padded layout in LDS, for workgroups that need
// each row's owner rank: pre[e] = the rows of the experts below e (counts
// taken as >= 0) and pre[E] = the valid row bound, each clamped to T_K.
// Thread i owns experts [i*kPer, i*kPer + kPer). Every thread of the
// workgroup calls it; it ends with a barrier.
template <int NT>
__device__ __forceinline__ void padded_prefix(const int* __restrict__ counts, int E, int T_K,
                                              int* pre, int* wave_tot, int tid, int lane,
                                              int wv) {
  constexpr int kPer = (kMaxPaddedE + NT - 1) / NT;
  int c[kPer];
  int mine = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int e = tid * kPer + q;
    c[q] = e < E ? max(counts[e], 0) : 0;
    mine += c[q];
  }
  int total;
  int ex = block_excl_scan<NT>(mine, lane, wv, wave_tot, total);  // syncs
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int e = tid * kPer + q;
    if (e < E) pre[e] = min(ex, T_K);
    ex += c[q];
  }
  if (tid == 0) pre[E] = min(total, T_K);
  __syncthreads();
}

template <int CPL>
__global__ __launch_bounds__(kRowWaves* kWave) void scatter_padded_scan_kernel(
    uint16_t* __restrict__ out, int T, const uint16_t* __restrict__ in, int T_K,
    const int* __restrict__ counts, int E, int EP, const int* __restrict__ ti, int D,
    int nsl) {
  constexpr int NT = kRowWaves * kWave;
  __shared__ int pre[kMaxPaddedE + 1];
  __shared__ int wave_tot[kRowWaves];
  __shared__ int stage[kRowWaves][kWave];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = uniform(tid >> 6);
  padded_prefix<NT>(counts, E, T_K, pre, wave_tot, tid, lane, wv);

  const int64_t unit = static_cast<int64_t>(blockIdx.x) * kRowWaves + wv;
  const int t = static_cast<int>(unit / nsl);
  const int sl = static_cast<int>(unit - static_cast<int64_t>(t) * nsl);
  if (t >= T) return;
  const int V = pre[E];
  int tv[kScanChunks];
#pragma unroll
  for (int q = 0; q < kScanChunks; ++q) {
    const int r = q * kWave + lane;
    tv[q] = r < V ? ti[r] : -1;
  }
  const int nch = D >> 3;
  const int slice0 = sl * kWave * CPL;
  uint16_t* orow = out + static_cast<int64_t>(t) * D;
  if (slice0 + kWave * CPL <= nch)
    padded_scan_reduce<CPL, true>(orow, in, T_K, pre, E, E / EP, tv, V, t, D, nch,
                                  slice0 + lane, lane, stage[wv]);
  else
    padded_scan_reduce<CPL, false>(orow, in, T_K, pre, E, E / EP, tv, V, t, D, nch,
                                   slice0 + lane, lane, stage[wv]);
}

// One (token, slice) of the by-token padded combine: the token's slots from
// the shuffle's inverse map, the valid rows sorted ascending, each then read
// from the slab of the rank that owns its expert; the additions and the
// early initial row are scatter_token's.
template <int CPL, int G, bool FULL>
__device__ __forceinline__ void scatter_padded_token(uint16_t* __restrict__ out,
                                                     const uint16_t* __restrict__ in, int T_K,
                                                     const int* pre, int E, int epr, int r,
                                                     int t, int K, int V, int D, int nch,
                                                     int base, int lane) {
  uint16_t* orow = out + static_cast<int64_t>(t) * D;
  const bool early = static_cast<int64_t>(t) * K < V;  // wave-uniform
  u32x4 o0[CPL];
  if (early) load_init<CPL, FULL>(o0, orow, nch, base);
  const bool ok = r >= 0 && r < V;
  const int n = __popcll(__ballot(ok));
  if (n == 0) return;
  const int sorted = wave_sort_asc(ok ? r : INT_MAX, lane, sort_width(uniform(K)));
  const int src = lane < n ? rank_of_row(pre, E, epr, sorted) * T_K + sorted : 0;
  if (!early) load_init<CPL, FULL>(o0, orow, nch, base);
  reduce_slice_from<CPL, G, FULL>(o0, orow, in, D, nch, base, src, n);
}

// The padded combine through row_of_pair: no row lists. Every workgroup
// first scans the expert counts into its LDS prefix (each row's owner rank,
// the valid bound V); the token's slots load meanwhile.
template <int CPL, int G>
__global__ __launch_bounds__(kRowWaves* kWave) void scatter_padded_tokens_kernel(
    uint16_t* __restrict__ out, int T, const uint16_t* __restrict__ in, int T_K,
    const int* __restrict__ counts, int E, int EP, const int* __restrict__ rop, int K, int D,
    int nsl) {
  constexpr int NT = kRowWaves * kWave;
  __shared__ int pre[kMaxPaddedE + 1];
  __shared__ int wave_tot[kRowWaves];
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wv = uniform(tid >> 6);
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * kRowWaves + wv;
  const int64_t t64 = unit / nsl;
  const int sl = static_cast<int>(unit - t64 * nsl);
  const bool live = t64 < T;  // wave-uniform; every wave joins the prefix scan
  const int t = live ? static_cast<int>(t64) : 0;
  const int r = (live && lane < K) ? rop[static_cast<int64_t>(t) * K + lane] : -1;
  padded_prefix<NT>(counts, E, T_K, pre, wave_tot, tid, lane, wv);
  if (!live) return;
  const int V = pre[E];
  const int nch = D >> 3;
  const int slice0 = sl * kWave * CPL;
  if (slice0 + kWave * CPL <= nch)
    scatter_padded_token<CPL, G, true>(out, in, T_K, pre, E, E / EP, r, t, K, V, D, nch,
                                       slice0 + lane, lane);
  else
    scatter_padded_token<CPL, G, false>(out, in, T_K, pre, E, E / EP, r, t, K, V, D, nch,
                                        slice0 + lane, lane);
}

size_t align256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// Rows in flight per group of the by-token combines: the next power of two
// >= K, at most 4 on a full grid (for K = 8 two groups of 4 measured 1.5 %
// faster than one of 8: fewer registers, more waves resident), 8 on a grid of
// at most kFewUnits waves, which is latency-bound and saves the second
// group's round trip.
constexpr int64_t kFewUnits = 4096;
int by_token_group(int K, int64_t units) {
  return K <= 1 ? 1 : (K <= 2 ? 2 : (K <= 4 || units > kFewUnits ? 4 : 8));
}

SliceShape combine_shape(int nch) {
  // kGroup rows * cpl chunks of loads are in flight per lane
  static const int allowed[] = {2, 4, 3, 1};
  return pick_slices(nch, allowed, 4, 1 << 20);
}

}  // namespace

// The one-workgroup CSR build applies.
bool small_build(int T, int a) { return a <= kSmallRows && T <= kSmallTok; }

// The two-launch CSR build applies (else the four-launch one).
bool two_launch_build(int T, int a) {
  return a <= kRangeMaxRows && (T + kRangeT - 1) / kRangeT <= kMaxRanges;
}

// start [T+1], then list [a] and, for the two-launch build, packed (row,
// token) pairs [a] and the [range][chunk] count and start matrices; for the
// four-launch build, slot [a].
size_t scatter_add_workspace_bytes(int T, int a) {
  const size_t head = align256((static_cast<size_t>(T) + 1) * sizeof(int)) +
                      align256(static_cast<size_t>(a) * sizeof(int));
  if (!two_launch_build(T, a)) return head + align256(static_cast<size_t>(a) * sizeof(int));
  const size_t nrange = (static_cast<size_t>(T) + kRangeT - 1) / kRangeT;
  const size_t G = (static_cast<size_t>(a) + kBucketRows - 1) / kBucketRows;
  return head + align256(static_cast<size_t>(a) * sizeof(int2)) +
         2 * align256(nrange * G * sizeof(int));
}

size_t scatter_add_padded_workspace_bytes(int T, int T_K, int E) {
  return align256((static_cast<size_t>(E) + 1) * sizeof(int)) +
         scatter_add_workspace_bytes(T, T_K);
}

namespace {

// Workspace layout of scatter_add_workspace_bytes(T, a) from `ws`: start
// [T+1], list [a], then slot [a] (four-launch build) or the two-launch
// build's buffers (see csr_two_launch).
void csr_layout(char* ws, int T, int a, int** start, int** list, int** slot) {
  *start = reinterpret_cast<int*>(ws);
  ws += align256((static_cast<size_t>(T) + 1) * sizeof(int));
  *list = reinterpret_cast<int*>(ws);
  ws += align256(static_cast<size_t>(a) * sizeof(int));
  *slot = reinterpret_cast<int*>(ws);
}

void csr_two_launch(const int* ti, int T, int a, const int* valid_rows, const int* counts, int E,
                    int* prefix, char* ws, int* start, int* list, hipStream_t stream) {
  const int nrange = (T + kRangeT - 1) / kRangeT;
  const int G = (a + kBucketRows - 1) / kBucketRows;
  char* p = ws + align256((static_cast<size_t>(T) + 1) * sizeof(int)) +
            align256(static_cast<size_t>(a) * sizeof(int));
  int2* packed = reinterpret_cast<int2*>(p);
  p += align256(static_cast<size_t>(a) * sizeof(int2));
  int* rcnt = reinterpret_cast<int*>(p);
  p += align256(static_cast<size_t>(nrange) * G * sizeof(int));
  int* roff = reinterpret_cast<int*>(p);
  hipLaunchKernelGGL(csr_bucket_kernel, dim3(G), dim3(kScanThreads), 0, stream, ti, T, a,
                     valid_rows, counts, E, prefix, nrange, G, rcnt, roff, packed);
  hipLaunchKernelGGL(csr_range_kernel, dim3(nrange), dim3(kRangeThreads), 0, stream, T, G,
                     rcnt, roff, packed, start, list);
}

}  // namespace

hipError_t launch_scatter_add_padded(const uint16_t* in, int EP, int T_K, const int* counts,
                                     int E, const int* ti, uint16_t* out, int T, int D,
                                     void* workspace, hipStream_t stream) {
  if (T_K <= kScanRows) {  // each wave finds its token's rows: no build
    const SliceShape sh = combine_shape(D / kChunk);
    const int64_t units = static_cast<int64_t>(T) * sh.nsl;
    const dim3 grid(static_cast<unsigned>((units + kRowWaves - 1) / kRowWaves));
#define LS(C)                                                                             \
  hipLaunchKernelGGL(scatter_padded_scan_kernel<C>, grid, dim3(kRowWaves * kWave), 0, stream, \
                     out, T, in, T_K, counts, E, EP, ti, D, sh.nsl)
    switch (sh.cpl) {
      case 1: LS(1); break;
      case 2: LS(2); break;
      case 3: LS(3); break;
      default: LS(4); break;
    }
#undef LS
    return hipGetLastError();
  }
  char* ws = static_cast<char*>(workspace);
  int* prefix = reinterpret_cast<int*>(ws);
  ws += align256((static_cast<size_t>(E) + 1) * sizeof(int));
  int* cnt = nullptr;
  int* list = nullptr;
  int* slot = nullptr;
  csr_layout(ws, T, T_K, &cnt, &list, &slot);
  if (small_build(T, T_K)) {
    hipLaunchKernelGGL(csr_small_kernel, dim3(1), dim3(kScanThreads), 0, stream, ti, T, T_K,
                       nullptr, counts, E, prefix, cnt, list);
  } else if (two_launch_build(T, T_K)) {
    csr_two_launch(ti, T, T_K, nullptr, counts, E, prefix, ws, cnt, list, stream);
  } else {
    hipLaunchKernelGGL(padded_prefix_kernel, dim3(1), dim3(kScanThreads), 0, stream, counts,
                       E, T_K, prefix);
    hipLaunchKernelGGL(csr_zero_kernel, dim3((T + 1 + 255) / 256), dim3(256), 0, stream, cnt,
                       T + 1);
    const dim3 rgrid((T_K + 255) / 256);
    hipLaunchKernelGGL(csr_count_kernel, rgrid, dim3(256), 0, stream, ti, T, T_K, prefix + E,
                       cnt, slot);
    hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, cnt, T);
    hipLaunchKernelGGL(csr_fill_kernel, rgrid, dim3(256), 0, stream, ti, T, T_K, prefix + E,
                       cnt, slot, list);
  }
  const SliceShape sh = combine_shape(D / kChunk);
  const int64_t units = static_cast<int64_t>(T) * sh.nsl;
  const dim3 grid(static_cast<unsigned>((units + kRowWaves - 1) / kRowWaves));
  const dim3 block(kRowWaves * kWave);
#define L(C)                                                                             \
  hipLaunchKernelGGL(scatter_padded_kernel<C>, grid, block, 0, stream, out, T, in, T_K, E, EP, \
                     prefix, cnt, list, D, sh.nsl)
  switch (sh.cpl) {
    case 1: L(1); break;
    case 2: L(2); break;
    case 3: L(3); break;
    default: L(4); break;
  }
#undef L
  return hipGetLastError();
}

hipError_t launch_scatter_add_padded_by_token(const uint16_t* in, int EP, int T_K,
                                              const int* counts, int E, const int* row_of_pair,
                                              int K, uint16_t* out, int T, int D,
                                              hipStream_t stream) {
  const SliceShape sh = combine_shape(D / kChunk);
  const int64_t units = static_cast<int64_t>(T) * sh.nsl;
  const int G = by_token_group(K, units);
  const dim3 grid(static_cast<unsigned>((units + kRowWaves - 1) / kRowWaves));
  const dim3 block(kRowWaves * kWave);
#define L2(C, GV)                                                                             \
  hipLaunchKernelGGL((scatter_padded_tokens_kernel<C, GV>), grid, block, 0, stream, out, T, in, \
                     T_K, counts, E, EP, row_of_pair, K, D, sh.nsl)
#define LG(C)                         \
  do {                                \
    if (G == 1) L2(C, 1);             \
    else if (G == 2) L2(C, 2);        \
    else if (G == 4) L2(C, 4);        \
    else L2(C, 8);                    \
  } while (0)
  switch (sh.cpl) {
    case 1: LG(1); break;
    case 2: LG(2); break;
    case 3: LG(3); break;
    default: LG(4); break;
  }
#undef LG
#undef L2
  return hipGetLastError();
}

hipError_t launch_scatter_add_by_token(uint16_t* out, int T, const uint16_t* in,
                                       const int* row_of_pair, int K, int a, int D,
                                       const int* valid_rows, hipStream_t stream) {
  const SliceShape sh = combine_shape(D / kChunk);
  const int64_t units = static_cast<int64_t>(T) * sh.nsl;
  const int G = by_token_group(K, units);
  const dim3 block(kRowWaves * kWave);
  // top-1 and top-2 on a full grid: kMultiTok tokens per wave (measured at
  // T=4096, D=5120, K=1: 2, 4 and 8 tokens against one; 4 the fastest, warm
  // and after a cache flush)
  if (K <= 2 && units > kFewUnits) {
    const int64_t mu = (static_cast<int64_t>(T) + kMultiTok - 1) / kMultiTok * sh.nsl;
    const dim3 mgrid(static_cast<unsigned>((mu + kRowWaves - 1) / kRowWaves));
#define LM(C)                                                                                  \
  do {                                                                                         \
    if (K <= 1)                                                                                \
      hipLaunchKernelGGL((scatter_tokens_multi_kernel<C, kMultiTok, 1>), mgrid, block, 0,      \
                         stream, out, T, in, row_of_pair, K, a, D, valid_rows, sh.nsl);        \
    else                                                                                       \
      hipLaunchKernelGGL((scatter_tokens_multi_kernel<C, kMultiTok, 2>), mgrid, block, 0,      \
                         stream, out, T, in, row_of_pair, K, a, D, valid_rows, sh.nsl);        \
  } while (0)
    switch (sh.cpl) {
      case 1: LM(1); break;
      case 2: LM(2); break;
      case 3: LM(3); break;
      default: LM(4); break;
    }
#undef LM
    return hipGetLastError();
  }
  const dim3 grid(static_cast<unsigned>((units + kRowWaves - 1) / kRowWaves));
#define L2(C, GV)                                                                          \
  hipLaunchKernelGGL((scatter_tokens_kernel<C, GV>), grid, block, 0, stream, out, T, in,  \
                     row_of_pair, K, a, D, valid_rows, sh.nsl)
#define LG(C)                         \
  do {                                \
    if (G == 1) L2(C, 1);             \
    else if (G == 2) L2(C, 2);        \
    else if (G == 4) L2(C, 4);        \
    else L2(C, 8);                    \
  } while (0)
  switch (sh.cpl) {
    case 1: LG(1); break;
    case 2: LG(2); break;
    case 3: LG(3); break;
    default: LG(4); break;
  }
#undef LG
#undef L2
  return hipGetLastError();
}

hipError_t launch_token_lists(const int* ti, int T, int a, const int* valid_rows,
                              void* workspace, const int** start, const int** list,
                              hipStream_t stream) {
  char* ws = static_cast<char*>(workspace);
  int* cnt = nullptr;  // [T+1]: counts, then starts
  int* lst = nullptr;
  int* slot = nullptr;
  csr_layout(ws, T, a, &cnt, &lst, &slot);
  *start = cnt;
  *list = lst;
  if (small_build(T, a)) {
    hipLaunchKernelGGL(csr_small_kernel, dim3(1), dim3(kScanThreads), 0, stream, ti, T, a,
                       valid_rows, nullptr, 0, nullptr, cnt, lst);
  } else if (two_launch_build(T, a)) {
    csr_two_launch(ti, T, a, valid_rows, nullptr, 0, nullptr, ws, cnt, lst, stream);
  } else {
    hipLaunchKernelGGL(csr_zero_kernel, dim3((T + 1 + 255) / 256), dim3(256), 0, stream, cnt,
                       T + 1);
    const dim3 rgrid((a + 255) / 256);
    hipLaunchKernelGGL(csr_count_kernel, rgrid, dim3(256), 0, stream, ti, T, a, valid_rows,
                       cnt, slot);
    hipLaunchKernelGGL(csr_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, cnt, T);
    hipLaunchKernelGGL(csr_fill_kernel, rgrid, dim3(256), 0, stream, ti, T, a, valid_rows,
                       cnt, slot, lst);
  }
  return hipGetLastError();
}

hipError_t launch_scatter_add(uint16_t* out, int T, const uint16_t* in, const int* ti,
                              int a, int D, const int* valid_rows, void* workspace,
                              hipStream_t stream) {
  const SliceShape sh = combine_shape(D / kChunk);
  const int64_t units = static_cast<int64_t>(T) * sh.nsl;
  const dim3 grid(static_cast<unsigned>((units + kRowWaves - 1) / kRowWaves));
  const dim3 block(kRowWaves * kWave);
  if (a <= kScanRows) {  // each wave finds its token's rows: no build
#define LS(C)                                                                             \
  hipLaunchKernelGGL(scatter_scan_kernel<C>, grid, block, 0, stream, out, T, in, ti, a, D, \
                     valid_rows, sh.nsl)
    switch (sh.cpl) {
      case 1: LS(1); break;
      case 2: LS(2); break;
      case 3: LS(3); break;
      default: LS(4); break;
    }
#undef LS
    return hipGetLastError();
  }
  const int* cnt;
  const int* list;
  const hipError_t e = launch_token_lists(ti, T, a, valid_rows, workspace, &cnt, &list, stream);
  if (e != hipSuccess) return e;
#define L(C)                                                                            \
  hipLaunchKernelGGL(scatter_csr_kernel<C>, grid, block, 0, stream, out, T, in, cnt, list, \
                     D, sh.nsl)
  switch (sh.cpl) {
    case 1: L(1); break;
    case 2: L(2); break;
    case 3: L(3); break;
    default: L(4); break;
  }
#undef L
  return hipGetLastError();
}

}  // namespace moe
