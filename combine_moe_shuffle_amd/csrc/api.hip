// C ABI of libmoe_shuffle.so: host-side argument checks, then the launchers.
// Every check runs before any HIP call, so a rejected call enqueues nothing
// (and these error paths run on a machine with no GPU).
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "moe_shuffle.h"
#include "launch.hpp"
#include "probe.hpp"

// The workspace of moe_shuffle_noalloc: a static device array, one copy per
// GPU. In host code `scratch` names a host-side stand-in, never a device
// address; the device address comes from hipGetSymbolAddress, taken once per
// device with that device current (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512];

moe_status_t fail(moe_status_t s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

moe_status_t ok() {
  g_err[0] = '\0';
  return MOE_OK;
}

moe_status_t hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;
constexpr int kMaxQuantD = 65536;     // 16 waves * 64 lanes * 8 chunks * 8
constexpr int kMaxFinalizeD = 65536;  // same bound for the finalize workgroup
constexpr int kMaxMhcD = 32768;       // 16 waves * 64 lanes * 4 chunks * 8
constexpr int kMaxMhcStreams = 4;

#define REQUIRE(cond, status, ...) \
  do {                             \
    if (!(cond)) return fail(status, __VA_ARGS__); \
  } while (0)

moe_status_t check_scores(const float* scores, int64_t st, int64_t se, int T, int E) {
  REQUIRE(E >= 1, MOE_ERR_INVALID_ARG, "E must be >= 1 (got %d)", E);
  REQUIRE(st >= 0 && se >= 0, MOE_ERR_INVALID_ARG, "score strides must be >= 0");
  if (T > 0) {
    REQUIRE(scores != nullptr, MOE_ERR_INVALID_ARG, "scores is NULL");
    REQUIRE(aligned(scores, 4), MOE_ERR_INVALID_ARG, "scores must be 4-byte aligned");
  }
  return MOE_OK;
}

moe_status_t check_rows(int D, int mult) {
  REQUIRE(D >= 0, MOE_ERR_INVALID_ARG, "D must be >= 0 (got %d)", D);
  REQUIRE(D % mult == 0, MOE_ERR_INVALID_ARG, "D must be a multiple of %d (got %d)", mult, D);
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(moe_status_t s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_err; }

size_t moe_shuffle_workspace_bytes(int32_t T, int32_t E, int32_t K) {
  if (T < 0 || E < 1 || K < 1) return 0;
  return moe::shuffle_workspace_bytes(T, E, K);
}

static moe_status_t check_shuffle(const float* scores, int64_t stride_t, int64_t stride_e,
                                  int32_t T, int32_t E, int32_t K, const int32_t* counts,
                                  const int32_t* expert_indices,
                                  const int32_t* token_indices) {
  REQUIRE(T >= 0, MOE_ERR_INVALID_ARG, "T must be >= 0 (got %d)", T);
  moe_status_t s = check_scores(scores, stride_t, stride_e, T, E);
  if (s != MOE_OK) return s;
  REQUIRE(K >= 1 && K <= E, MOE_ERR_INVALID_ARG, "K must be in [1, E] (K=%d, E=%d)", K, E);
  REQUIRE(E <= kMaxE, MOE_ERR_UNSUPPORTED, "E > %d is not supported (got %d)", kMaxE, E);
  REQUIRE(K <= kMaxK, MOE_ERR_UNSUPPORTED, "K > %d is not supported (got %d)", kMaxK, K);
  REQUIRE(static_cast<int64_t>(T) * K < (int64_t{1} << 31), MOE_ERR_INVALID_ARG,
          "T*K must be < 2^31");
  REQUIRE(counts != nullptr, MOE_ERR_INVALID_ARG, "counts is NULL");
  if (T > 0)
    REQUIRE(expert_indices && token_indices, MOE_ERR_INVALID_ARG, "index outputs are NULL");
  return MOE_OK;
}

moe_status_t moe_shuffle(const float* scores, int64_t stride_t, int64_t stride_e, int32_t T,
                         int32_t E, int32_t K, const int32_t* valid_token_count,
                         int32_t* counts, int32_t* expert_indices, int32_t* token_indices,
                         int32_t* row_of_pair, void* workspace, size_t workspace_bytes,
                         void* stream) {
  moe_status_t s =
      check_shuffle(scores, stride_t, stride_e, T, E, K, counts, expert_indices, token_indices);
  if (s != MOE_OK) return s;
  if (T > 0) {
    const size_t need = moe::shuffle_workspace_bytes(T, E, K);
    REQUIRE(workspace != nullptr && workspace_bytes >= need, MOE_ERR_WORKSPACE,
            "shuffle workspace needs %zu bytes (got %zu)", need, workspace_bytes);
    REQUIRE(aligned(workspace, 256), MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  }
  // T == 0 still writes counts (all zero)
  return hip_status(moe::launch_shuffle(scores, stride_t, stride_e, T, E, K, valid_token_count,
                                        counts, expert_indices, token_indices, row_of_pair,
                                        workspace, static_cast<hipStream_t>(stream)),
                    "moe_shuffle");
}

}  // extern "C"

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch`, per device

// The device address of this GPU's copy of `scratch`, where GPU = the
// current device, which must also be the stream's. Taken once per device.
moe_status_t noalloc_scratch(void* stream, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess)
      return fail(MOE_ERR_HIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    REQUIRE(sdev == dev, MOE_ERR_INVALID_ARG,
            "the stream belongs to device %d but the current device is %d", sdev, dev);
  }
  REQUIRE(dev >= 0 && dev < kMaxScratchDevices, MOE_ERR_UNSUPPORTED,
          "device %d is beyond the %d devices the static scratch serves", dev,
          kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_shuffle_noalloc(const float* scores, int64_t stride_t, int64_t stride_e,
                                 int32_t T, int32_t E, int32_t K,
                                 const int32_t* valid_token_count, int32_t* counts,
                                 int32_t* expert_indices, int32_t* token_indices,
                                 int32_t* row_of_pair, void* stream) {
  moe_status_t s =
      check_shuffle(scores, stride_t, stride_e, T, E, K, counts, expert_indices, token_indices);
  if (s != MOE_OK) return s;
  void* ws = nullptr;
  if (T > 0) {
    const size_t need = moe::shuffle_workspace_bytes(T, E, K);
    REQUIRE(need <= MOE_NOALLOC_SCRATCH_BYTES, MOE_ERR_WORKSPACE,
            "moe_shuffle_noalloc: T=%d, E=%d, K=%d need %zu bytes of scratch, more than the "
            "%zu the library holds",
            T, E, K, need, static_cast<size_t>(MOE_NOALLOC_SCRATCH_BYTES));
    s = noalloc_scratch(stream, &ws);
    if (s != MOE_OK) return s;
  }
  // T == 0 only writes counts (all zero) and touches no scratch
  return hip_status(moe::launch_shuffle(scores, stride_t, stride_e, T, E, K, valid_token_count,
                                        counts, expert_indices, token_indices, row_of_pair, ws,
                                        static_cast<hipStream_t>(stream)),
                    "moe_shuffle_noalloc");
}

static moe_status_t check_gather(const moe_bf16_t* x, int32_t T, int32_t D, int32_t a,
                                 const float* scores, int64_t st, int64_t se, int32_t E,
                                 const void* out, int out_align) {
  REQUIRE(T >= 0 && a >= 0, MOE_ERR_INVALID_ARG, "T and a must be >= 0");
  moe_status_t s = check_rows(D, 8);
  if (s != MOE_OK) return s;
  if (a == 0 || D == 0) return MOE_OK;
  s = check_scores(scores, st, se, 1, E);
  if (s != MOE_OK) return s;
  REQUIRE(x != nullptr || T == 0, MOE_ERR_INVALID_ARG, "x is NULL");
  REQUIRE(out != nullptr, MOE_ERR_INVALID_ARG, "out is NULL");
  REQUIRE(aligned(x, 16), MOE_ERR_INVALID_ARG, "x must be 16-byte aligned");
  REQUIRE(aligned(out, out_align), MOE_ERR_INVALID_ARG, "out must be %d-byte aligned",
          out_align);
  return MOE_OK;
}

size_t moe_gather_scale_workspace_bytes(int32_t T, int32_t a) {
  if (T < 0 || a < 0) return 0;
  return moe::scatter_add_workspace_bytes(T, a);
}

moe_status_t moe_gather_scale(const moe_bf16_t* x, int32_t T, int32_t D,
                              const int32_t* token_indices, const int32_t* expert_indices,
                              int32_t a, const float* scores, int64_t stride_t,
                              int64_t stride_e, int32_t E, const int32_t* valid_rows,
                              moe_bf16_t* out, void* workspace, size_t workspace_bytes,
                              void* stream) {
  moe_status_t s = check_gather(x, T, D, a, scores, stride_t, stride_e, E, out, 16);
  if (s != MOE_OK) return s;
  if (a == 0 || D == 0) return ok();
  REQUIRE(token_indices && expert_indices, MOE_ERR_INVALID_ARG, "index inputs are NULL");
  if (workspace != nullptr) {
    const size_t need = moe::scatter_add_workspace_bytes(T, a);
    REQUIRE(workspace_bytes >= need, MOE_ERR_WORKSPACE,
            "gather_scale workspace needs %zu bytes (got %zu)", need, workspace_bytes);
    REQUIRE(aligned(workspace, 256), MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  }
  if (T == 0) return ok();  // no token row exists, so no row is written
  return hip_status(moe::launch_gather_scale(x, T, D, token_indices, expert_indices, a, scores,
                                             stride_t, stride_e, E, valid_rows, out, workspace,
                                             static_cast<hipStream_t>(stream)),
                    "moe_gather_scale");
}

moe_status_t moe_gather_scale_by_token(const moe_bf16_t* x, int32_t T, int32_t D,
                                       const int32_t* row_of_pair, int32_t K,
                                       const int32_t* expert_indices, int32_t a,
                                       const float* scores, int64_t stride_t,
                                       int64_t stride_e, int32_t E,
                                       const int32_t* valid_rows, moe_bf16_t* out,
                                       void* stream) {
  moe_status_t s = check_gather(x, T, D, a, scores, stride_t, stride_e, E, out, 16);
  if (s != MOE_OK) return s;
  REQUIRE(K >= 1 && K <= kMaxK, MOE_ERR_INVALID_ARG, "K must be in [1, %d] (got %d)", kMaxK, K);
  if (a == 0 || D == 0 || T == 0) return ok();
  REQUIRE(row_of_pair && expert_indices, MOE_ERR_INVALID_ARG, "index inputs are NULL");
  return hip_status(moe::launch_gather_scale_by_token(x, T, D, row_of_pair, K, expert_indices,
                                                      a, scores, stride_t, stride_e, E,
                                                      valid_rows, out,
                                                      static_cast<hipStream_t>(stream)),
                    "moe_gather_scale_by_token");
}

moe_status_t moe_gather_scale_quant(const moe_bf16_t* x, int32_t T, int32_t D,
                                    const int32_t* token_indices,
                                    const int32_t* expert_indices, int32_t a,
                                    const float* scores, int64_t stride_t, int64_t stride_e,
                                    int32_t E, const float* scale_ub,
                                    const int32_t* valid_rows, uint8_t* out_fp8,
                                    float* out_scale, void* stream) {
  moe_status_t s = check_gather(x, T, D, a, scores, stride_t, stride_e, E, out_fp8, 16);
  if (s != MOE_OK) return s;
  if (a == 0 || D == 0) return ok();
  REQUIRE(D <= kMaxQuantD, MOE_ERR_UNSUPPORTED, "D > %d is not supported (got %d)", kMaxQuantD,
          D);
  REQUIRE(token_indices && expert_indices, MOE_ERR_INVALID_ARG, "index inputs are NULL");
  REQUIRE(out_scale != nullptr && aligned(out_scale, 4), MOE_ERR_INVALID_ARG,
          "out_scale is NULL or misaligned");
  REQUIRE(scale_ub == nullptr || aligned(scale_ub, 4), MOE_ERR_INVALID_ARG,
          "scale_ub misaligned");
  return hip_status(moe::launch_gather_scale_quant(x, T, D, token_indices, expert_indices, a,
                                                   scores, stride_t, stride_e, E, scale_ub,
                                                   valid_rows, out_fp8, out_scale,
                                                   static_cast<hipStream_t>(stream)),
                    "moe_gather_scale_quant");
}

size_t moe_scatter_add_workspace_bytes(int32_t T, int32_t a) {
  if (T < 0 || a < 0) return 0;
  return moe::scatter_add_workspace_bytes(T, a);
}

static moe_status_t check_scatter(const moe_bf16_t* out, int32_t T, const moe_bf16_t* in,
                                  int32_t a, int32_t D) {
  REQUIRE(T >= 0 && a >= 0, MOE_ERR_INVALID_ARG, "T and a must be >= 0");
  moe_status_t s = check_rows(D, 8);
  if (s != MOE_OK) return s;
  if (a == 0 || D == 0 || T == 0) return MOE_OK;
  REQUIRE(out && in, MOE_ERR_INVALID_ARG, "out_tokens or in_tokens is NULL");
  REQUIRE(aligned(out, 16) && aligned(in, 16), MOE_ERR_INVALID_ARG,
          "row buffers must be 16-byte aligned");
  return MOE_OK;
}

moe_status_t moe_scatter_add(moe_bf16_t* out_tokens, int32_t T, const moe_bf16_t* in_tokens,
                             const int32_t* token_indices, int32_t a, int32_t D,
                             const int32_t* valid_rows, void* workspace,
                             size_t workspace_bytes, void* stream) {
  moe_status_t s = check_scatter(out_tokens, T, in_tokens, a, D);
  if (s != MOE_OK) return s;
  if (a == 0 || D == 0 || T == 0) return ok();
  REQUIRE(token_indices != nullptr, MOE_ERR_INVALID_ARG, "token_indices is NULL");
  const size_t need = moe::scatter_add_workspace_bytes(T, a);
  REQUIRE(workspace != nullptr && workspace_bytes >= need, MOE_ERR_WORKSPACE,
          "scatter_add workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  REQUIRE(aligned(workspace, 256), MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return hip_status(moe::launch_scatter_add(out_tokens, T, in_tokens, token_indices, a, D,
                                            valid_rows, workspace,
                                            static_cast<hipStream_t>(stream)),
                    "moe_scatter_add");
}

moe_status_t moe_scatter_add_by_token(moe_bf16_t* out_tokens, int32_t T,
                                      const moe_bf16_t* in_tokens, const int32_t* row_of_pair,
                                      int32_t K, int32_t a, int32_t D,
                                      const int32_t* valid_rows, void* stream) {
  moe_status_t s = check_scatter(out_tokens, T, in_tokens, a, D);
  if (s != MOE_OK) return s;
  REQUIRE(K >= 1 && K <= kMaxK, MOE_ERR_INVALID_ARG, "K must be in [1, %d] (got %d)", kMaxK, K);
  if (a == 0 || D == 0 || T == 0) return ok();
  REQUIRE(row_of_pair != nullptr, MOE_ERR_INVALID_ARG, "row_of_pair is NULL");
  return hip_status(moe::launch_scatter_add_by_token(out_tokens, T, in_tokens, row_of_pair, K,
                                                     a, D, valid_rows,
                                                     static_cast<hipStream_t>(stream)),
                    "moe_scatter_add_by_token");
}

size_t moe_scatter_add_padded_workspace_bytes(int32_t T, int32_t T_K, int32_t E) {
  if (T < 0 || T_K < 0 || E < 1) return 0;
  return moe::scatter_add_padded_workspace_bytes(T, T_K, E);
}

moe_status_t moe_scatter_add_padded(const moe_bf16_t* in_tokens, int32_t EP, int32_t T_K,
                                    const int32_t* token_counts, int32_t E,
                                    const int32_t* token_indices, moe_bf16_t* out_tokens,
                                    int32_t T, int32_t D, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  REQUIRE(EP >= 1 && E >= 1 && T_K >= 0 && T >= 0, MOE_ERR_INVALID_ARG,
          "EP, E >= 1 and T_K, T >= 0 required (EP=%d E=%d T_K=%d T=%d)", EP, E, T_K, T);
  REQUIRE(E % EP == 0, MOE_ERR_INVALID_ARG, "E must be a multiple of EP (E=%d, EP=%d)", E, EP);
  REQUIRE(E <= kMaxE, MOE_ERR_UNSUPPORTED, "E > %d is not supported (got %d)", kMaxE, E);
  REQUIRE(static_cast<int64_t>(EP) * T_K < (int64_t{1} << 31), MOE_ERR_INVALID_ARG,
          "EP*T_K must be < 2^31");
  moe_status_t s = check_scatter(out_tokens, T, in_tokens, T_K, D);
  if (s != MOE_OK) return s;
  if (T_K == 0 || D == 0 || T == 0) return ok();
  REQUIRE(token_counts && token_indices, MOE_ERR_INVALID_ARG, "index inputs are NULL");
  const size_t need = moe::scatter_add_padded_workspace_bytes(T, T_K, E);
  REQUIRE(workspace != nullptr && workspace_bytes >= need, MOE_ERR_WORKSPACE,
          "scatter_add_padded workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  REQUIRE(aligned(workspace, 256), MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return hip_status(moe::launch_scatter_add_padded(in_tokens, EP, T_K, token_counts, E,
                                                   token_indices, out_tokens, T, D, workspace,
                                                   static_cast<hipStream_t>(stream)),
                    "moe_scatter_add_padded");
}

moe_status_t moe_scatter_add_padded_by_token(const moe_bf16_t* in_tokens, int32_t EP,
                                             int32_t T_K, const int32_t* token_counts,
                                             int32_t E, const int32_t* row_of_pair, int32_t K,
                                             moe_bf16_t* out_tokens, int32_t T, int32_t D,
                                             void* stream) {
  REQUIRE(EP >= 1 && E >= 1 && T_K >= 0 && T >= 0, MOE_ERR_INVALID_ARG,
          "EP, E >= 1 and T_K, T >= 0 required (EP=%d E=%d T_K=%d T=%d)", EP, E, T_K, T);
  REQUIRE(E % EP == 0, MOE_ERR_INVALID_ARG, "E must be a multiple of EP (E=%d, EP=%d)", E, EP);
  REQUIRE(E <= kMaxE, MOE_ERR_UNSUPPORTED, "E > %d is not supported (got %d)", kMaxE, E);
  REQUIRE(static_cast<int64_t>(EP) * T_K < (int64_t{1} << 31), MOE_ERR_INVALID_ARG,
          "EP*T_K must be < 2^31");
  REQUIRE(K >= 1 && K <= kMaxK, MOE_ERR_INVALID_ARG, "K must be in [1, %d] (got %d)", kMaxK, K);
  moe_status_t s = check_scatter(out_tokens, T, in_tokens, T_K, D);
  if (s != MOE_OK) return s;
  if (T_K == 0 || D == 0 || T == 0) return ok();
  REQUIRE(token_counts && row_of_pair, MOE_ERR_INVALID_ARG, "index inputs are NULL");
  return hip_status(moe::launch_scatter_add_padded_by_token(in_tokens, EP, T_K, token_counts,
                                                            E, row_of_pair, K, out_tokens, T, D,
                                                            static_cast<hipStream_t>(stream)),
                    "moe_scatter_add_padded_by_token");
}

size_t moe_shuffling_workspace_bytes(int32_t EP, int32_t n_local, int64_t em_rows) {
  if (EP < 1 || n_local < 0 || em_rows < 0) return 0;
  return moe::shuffling_workspace_bytes(EP * n_local, em_rows);
}

static moe_status_t shuffling(bool inverse, const moe_bf16_t* in, int64_t in_rows,
                              moe_bf16_t* out, int64_t out_rows, int32_t D,
                              const int32_t* counts, int32_t EP, int32_t C, int32_t c_lo,
                              int32_t c_hi, int64_t rank_stride, int32_t* out_counts,
                              void* workspace, size_t workspace_bytes, void* stream) {
  const char* what = inverse ? "moe_split_shuffling" : "moe_combine_shuffling";
  REQUIRE(EP >= 1 && EP <= moe::kMaxShufflingRanks, MOE_ERR_UNSUPPORTED,
          "%s: EP must be in [1, %d] (got %d)", what, moe::kMaxShufflingRanks, EP);
  REQUIRE(C >= 1 && c_lo >= 0 && c_lo <= c_hi && c_hi <= C, MOE_ERR_INVALID_ARG,
          "%s: need 0 <= c_lo <= c_hi <= C, C >= 1 (C=%d c_lo=%d c_hi=%d)", what, C, c_lo, c_hi);
  REQUIRE(static_cast<int64_t>(c_hi - c_lo) * EP <= moe::kMaxShufflingSegments,
          MOE_ERR_UNSUPPORTED, "%s: (c_hi - c_lo) * EP > %d", what,
          moe::kMaxShufflingSegments);
  REQUIRE(in_rows >= 0 && out_rows >= 0 && in_rows < (int64_t{1} << 31) &&
              out_rows < (int64_t{1} << 31),
          MOE_ERR_INVALID_ARG, "%s: row counts must be in [0, 2^31)", what);
  REQUIRE(rank_stride < 0 || static_cast<int64_t>(EP) * rank_stride < (int64_t{1} << 31),
          MOE_ERR_INVALID_ARG, "%s: EP * rank_stride must be < 2^31", what);
  moe_status_t s = check_rows(D, 8);
  if (s != MOE_OK) return s;
  REQUIRE(counts != nullptr, MOE_ERR_INVALID_ARG, "%s: counts is NULL", what);
  REQUIRE(inverse || out_counts != nullptr, MOE_ERR_INVALID_ARG, "%s: out_counts is NULL",
          what);
  REQUIRE((in_rows == 0 || in) && (out_rows == 0 || out), MOE_ERR_INVALID_ARG,
          "%s: row buffer is NULL", what);
  REQUIRE(aligned(in, 16) && aligned(out, 16), MOE_ERR_INVALID_ARG,
          "%s: row buffers must be 16-byte aligned", what);
  const int64_t em_rows = inverse ? in_rows : out_rows;
  const size_t need = moe::shuffling_workspace_bytes((c_hi - c_lo) * EP, em_rows);
  REQUIRE(workspace != nullptr && workspace_bytes >= need, MOE_ERR_WORKSPACE,
          "%s workspace needs %zu bytes (got %zu)", what, need, workspace_bytes);
  REQUIRE(aligned(workspace, 256), MOE_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return hip_status(moe::launch_shuffling(inverse, in, in_rows, out, out_rows, D, counts, EP, C,
                                          c_lo, c_hi, rank_stride, out_counts, workspace,
                                          static_cast<hipStream_t>(stream)),
                    what);
}

moe_status_t moe_combine_shuffling(const moe_bf16_t* in, int64_t in_rows, moe_bf16_t* out,
                                   int64_t out_rows, int32_t D, const int32_t* counts,
                                   int32_t EP, int32_t C, int32_t c_lo, int32_t c_hi,
                                   int64_t rank_stride, int32_t* out_counts, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return shuffling(false, in, in_rows, out, out_rows, D, counts, EP, C, c_lo, c_hi,
                   rank_stride, out_counts, workspace, workspace_bytes, stream);
}

moe_status_t moe_split_shuffling(const moe_bf16_t* in, int64_t in_rows, moe_bf16_t* out,
                                 int64_t out_rows, int32_t D, const int32_t* counts, int32_t EP,
                                 int32_t C, int32_t c_lo, int32_t c_hi, int64_t rank_stride,
                                 int32_t* out_counts, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return shuffling(true, in, in_rows, out, out_rows, D, counts, EP, C, c_lo, c_hi,
                   rank_stride, out_counts, workspace, workspace_bytes, stream);
}

size_t moe_mxfp8_scale_bytes(int32_t M, int32_t D, uint32_t flags) {
  if (M < 0 || D < 0) return 0;
  const size_t cols = static_cast<size_t>(D) / 32;
  if (!(flags & MOE_FINALIZE_MX_SWIZZLED)) return static_cast<size_t>(M) * cols;
  return (static_cast<size_t>(M) + 127) / 128 * 128 * ((cols + 3) / 4 * 4);
}

moe_status_t moe_finalize_rmsnorm(const moe_bf16_t* y_permuted, int64_t rows,
                                  const void* expert_weights, const int32_t* row_of_pair,
                                  const moe_bf16_t* shared, const moe_bf16_t* gamma, float eps,
                                  int32_t T, int32_t K, int32_t D, uint32_t flags,
                                  moe_bf16_t* out, uint8_t* mx_codes, uint8_t* mx_scales,
                                  void* stream) {
  REQUIRE(T >= 0 && rows >= 0, MOE_ERR_INVALID_ARG, "T and rows must be >= 0");
  REQUIRE(K >= 1, MOE_ERR_INVALID_ARG, "K must be >= 1 (got %d)", K);
  REQUIRE(K <= kMaxK, MOE_ERR_UNSUPPORTED, "K > %d is not supported (got %d)", kMaxK, K);
  constexpr uint32_t kKnown =
      MOE_FINALIZE_BF16_SQUARES | MOE_FINALIZE_BF16_WEIGHTS | MOE_FINALIZE_MX_SWIZZLED;
  REQUIRE((flags & ~kKnown) == 0, MOE_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  REQUIRE((mx_codes == nullptr) == (mx_scales == nullptr), MOE_ERR_INVALID_ARG,
          "mx_codes and mx_scales must both be NULL or both be set");
  REQUIRE(!(flags & MOE_FINALIZE_MX_SWIZZLED) || mx_codes != nullptr, MOE_ERR_INVALID_ARG,
          "the swizzled scale layout needs MXFP8 outputs");
  moe_status_t s = check_rows(D, (flags & MOE_FINALIZE_MX_SWIZZLED) ? 128 : (mx_codes ? 32 : 8));
  if (s != MOE_OK) return s;
  REQUIRE(D <= kMaxFinalizeD, MOE_ERR_UNSUPPORTED, "D > %d is not supported (got %d)",
          kMaxFinalizeD, D);
  if (T == 0 || D == 0) return ok();
  REQUIRE(expert_weights && row_of_pair && gamma && out, MOE_ERR_INVALID_ARG,
          "a required pointer is NULL");
  REQUIRE(y_permuted != nullptr || rows == 0, MOE_ERR_INVALID_ARG, "y_permuted is NULL");
  REQUIRE(aligned(y_permuted, 16) && aligned(gamma, 16) && aligned(out, 16) &&
              aligned(shared, 16) && aligned(mx_codes, 16),
          MOE_ERR_INVALID_ARG, "row buffers must be 16-byte aligned");
  REQUIRE(aligned(expert_weights, (flags & MOE_FINALIZE_BF16_WEIGHTS) ? 2 : 4) &&
              aligned(row_of_pair, 4),
          MOE_ERR_INVALID_ARG, "expert_weights / row_of_pair misaligned");
  return hip_status(moe::launch_finalize_rmsnorm(y_permuted, rows, expert_weights, row_of_pair,
                                                 shared, gamma, eps, T, K, D, flags, out,
                                                 mx_codes, mx_scales,
                                                 static_cast<hipStream_t>(stream)),
                    "moe_finalize_rmsnorm");
}

moe_status_t moe_finalize_mhc(const moe_bf16_t* y_permuted, int64_t rows,
                              const void* expert_weights, const int32_t* row_of_pair,
                              const moe_bf16_t* shared, const moe_bf16_t* residual,
                              const float* post, const float* comb, const float* pre,
                              const moe_bf16_t* gamma, float eps, int32_t T, int32_t K, int32_t D,
                              int32_t hc, uint32_t flags, moe_bf16_t* residual_out,
                              moe_bf16_t* out, uint8_t* mx_codes, uint8_t* mx_scales,
                              void* stream) {
  REQUIRE(T >= 0 && rows >= 0, MOE_ERR_INVALID_ARG, "T and rows must be >= 0");
  REQUIRE(K >= 1, MOE_ERR_INVALID_ARG, "K must be >= 1 (got %d)", K);
  REQUIRE(K <= kMaxK, MOE_ERR_UNSUPPORTED, "K > %d is not supported (got %d)", kMaxK, K);
  REQUIRE(hc >= 1, MOE_ERR_INVALID_ARG, "hc must be >= 1 (got %d)", hc);
  REQUIRE(hc <= kMaxMhcStreams, MOE_ERR_UNSUPPORTED, "hc > %d is not supported (got %d)",
          kMaxMhcStreams, hc);
  constexpr uint32_t kKnown =
      MOE_FINALIZE_BF16_SQUARES | MOE_FINALIZE_BF16_WEIGHTS | MOE_FINALIZE_MX_SWIZZLED;
  REQUIRE((flags & ~kKnown) == 0, MOE_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  REQUIRE((mx_codes == nullptr) == (mx_scales == nullptr), MOE_ERR_INVALID_ARG,
          "mx_codes and mx_scales must both be NULL or both be set");
  REQUIRE(pre != nullptr || (mx_codes == nullptr && out == nullptr), MOE_ERR_INVALID_ARG,
          "without pre (residual only) out and the MXFP8 outputs must be NULL");
  REQUIRE(!(flags & MOE_FINALIZE_MX_SWIZZLED) || mx_codes != nullptr, MOE_ERR_INVALID_ARG,
          "the swizzled scale layout needs MXFP8 outputs");
  moe_status_t s = check_rows(D, (flags & MOE_FINALIZE_MX_SWIZZLED) ? 128 : (mx_codes ? 32 : 8));
  if (s != MOE_OK) return s;
  REQUIRE(D <= kMaxMhcD, MOE_ERR_UNSUPPORTED, "D > %d is not supported (got %d)", kMaxMhcD, D);
  if (T == 0 || D == 0) return ok();
  REQUIRE(expert_weights && row_of_pair && residual && post && comb && residual_out,
          MOE_ERR_INVALID_ARG, "a required pointer is NULL");
  REQUIRE(pre == nullptr || (gamma != nullptr && out != nullptr), MOE_ERR_INVALID_ARG,
          "gamma and out are required with pre");
  REQUIRE(y_permuted != nullptr || rows == 0, MOE_ERR_INVALID_ARG, "y_permuted is NULL");
  REQUIRE(aligned(y_permuted, 16) && aligned(gamma, 16) && aligned(out, 16) &&
              aligned(shared, 16) && aligned(mx_codes, 16) && aligned(residual, 16) &&
              aligned(residual_out, 16),
          MOE_ERR_INVALID_ARG, "row buffers must be 16-byte aligned");
  REQUIRE(aligned(expert_weights, (flags & MOE_FINALIZE_BF16_WEIGHTS) ? 2 : 4) &&
              aligned(row_of_pair, 4) && aligned(post, 4) && aligned(comb, 4) &&
              aligned(pre, 4),
          MOE_ERR_INVALID_ARG, "weights, row_of_pair or mix coefficients misaligned");
  return hip_status(moe::launch_finalize_mhc(y_permuted, rows, expert_weights, row_of_pair,
                                             shared, residual, post, comb, pre, gamma, eps, T,
                                             K, D, hc, flags, residual_out, out, mx_codes,
                                             mx_scales, static_cast<hipStream_t>(stream)),
                    "moe_finalize_mhc");
}

moe_status_t moe_convert_check(const float* in, int64_t n, moe_bf16_t* bf16_out,
                               uint8_t* e4m3_out, void* stream) {
  REQUIRE(n >= 0, MOE_ERR_INVALID_ARG, "n must be >= 0");
  if (n == 0) return ok();
  REQUIRE(in != nullptr && aligned(in, 4), MOE_ERR_INVALID_ARG, "in is NULL or misaligned");
  REQUIRE(n < (int64_t{1} << 31) * 256, MOE_ERR_INVALID_ARG, "n too large");
  return hip_status(moe::launch_convert_check(in, n, bf16_out, e4m3_out,
                                              static_cast<hipStream_t>(stream)),
                    "moe_convert_check");
}

int32_t moe_launch_floor_threads(int32_t T, int32_t D) {
  if (T < 1 || D < 8 || D % 8 != 0 || D > kMaxFinalizeD) return 0;
  return moe::launch_floor_threads(T, D);
}

moe_status_t moe_launch_floor(int32_t kind, int32_t T, int32_t D, const void* src, int32_t* dst,
                              void* stream) {
  REQUIRE(kind == 0 || kind == 1, MOE_ERR_INVALID_ARG, "kind must be 0 or 1 (got %d)", kind);
  REQUIRE(T >= 1 && T <= (1 << 20), MOE_ERR_INVALID_ARG, "T must be in [1, 2^20] (got %d)", T);
  REQUIRE(D >= 8 && D % 8 == 0 && D <= kMaxFinalizeD, MOE_ERR_INVALID_ARG,
          "D must be a multiple of 8 in [8, %d] (got %d)", kMaxFinalizeD, D);
  if (kind == 1) {
    REQUIRE(src != nullptr && dst != nullptr, MOE_ERR_INVALID_ARG, "src and dst are required");
    REQUIRE(aligned(src, 16) && aligned(dst, 4), MOE_ERR_INVALID_ARG, "src or dst misaligned");
  }
  return hip_status(moe::launch_floor(kind, T, D, src, dst, static_cast<hipStream_t>(stream)),
                    "moe_launch_floor");
}

moe_status_t moe_stream_probe(int32_t layout, int32_t R, int32_t W, int64_t units,
                              const void* src, void* dst, void* stream) {
  REQUIRE(layout == 0 || layout == 1, MOE_ERR_INVALID_ARG, "layout must be 0 or 1 (got %d)",
          layout);
  REQUIRE(R >= 1 && R <= moe::kStreamMaxR, MOE_ERR_INVALID_ARG, "R must be in [1, %d] (got %d)",
          moe::kStreamMaxR, R);
  REQUIRE(W >= 1 && W <= moe::kStreamMaxW, MOE_ERR_INVALID_ARG, "W must be in [1, %d] (got %d)",
          moe::kStreamMaxW, W);
  REQUIRE(units >= 0 && units < (int64_t{1} << 31), MOE_ERR_INVALID_ARG,
          "units must be in [0, 2^31)");
  if (units == 0) return ok();
  REQUIRE(src != nullptr && dst != nullptr, MOE_ERR_INVALID_ARG, "src and dst are required");
  REQUIRE(aligned(src, 16) && aligned(dst, 16), MOE_ERR_INVALID_ARG,
          "src and dst must be 16-byte aligned");
  const uintptr_t s0 = reinterpret_cast<uintptr_t>(src), d0 = reinterpret_cast<uintptr_t>(dst);
  const uintptr_t s1 = s0 + static_cast<uintptr_t>(units) * R * 1024;
  const uintptr_t d1 = d0 + static_cast<uintptr_t>(units) * W * 1024;
  REQUIRE(s1 <= d0 || d1 <= s0, MOE_ERR_INVALID_ARG, "src and dst overlap");
  return hip_status(moe::launch_stream_probe(layout, R, W, units, src, dst,
                                             static_cast<hipStream_t>(stream)),
                    "moe_stream_probe");
}

}  // extern "C"
