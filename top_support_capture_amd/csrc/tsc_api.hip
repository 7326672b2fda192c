// Host side of the C ABI declared in include/tsc.h: argument validation and kernel launch on the
// caller's stream. Nothing here allocates device memory or synchronizes.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "tsc.h"
#include "tsc_fast.h"
#include "tsc_csr.h"
#include "tsc_replay.h"

namespace {

constexpr int32_t kVersion = 100;  // 0.1.0

// The dynamic LDS limit of a kernel is a per-device attribute: it is set once for each device
// the calling thread has current when it launches (devices 0..kMaxDevices-1).
constexpr int kMaxDevices = 64;

// One workgroup per row. Rows the single-read path serves run there; every other row runs the
// general multi-pass algorithm inside the same launch.
template <int DT, bool BITS>
hipError_t launch_sampler(const tsc::SampleArgs& a, hipStream_t stream) {
  static std::mutex mu;
  static bool attr_set[kMaxDevices] = {};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  {
    std::lock_guard<std::mutex> lock(mu);
    if (!attr_set[dev]) {
      err = hipFuncSetAttribute(reinterpret_cast<const void*>(&tsc::sample_fast_kernel<DT, BITS>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)tsc::kFastDynLds);
      if (err != hipSuccess) return err;
      attr_set[dev] = true;
    }
  }
  hipLaunchKernelGGL((tsc::sample_fast_kernel<DT, BITS>), dim3((unsigned)a.B), dim3(tsc::kThreads),
                     tsc::kFastDynLds, stream, a);
  return hipGetLastError();
}

// Limit of the bounded waits between the waves of a workgroup (tsc_set_wait_limit).
std::atomic<uint32_t> g_wait_limit{tsc::kDefaultWaitLimit};

// Packed slots past each length filled with -1 / NaN after a capture (tsc_set_debug_poison).
#ifdef TSC_DEBUG_POISON
std::atomic<int32_t> g_poison{1};
#else
std::atomic<int32_t> g_poison{0};
#endif

}  // namespace

extern "C" {

int32_t tsc_version(void) { return kVersion; }

int32_t tsc_set_debug_poison(int32_t on) {
  return g_poison.exchange(on != 0 ? 1 : 0, std::memory_order_relaxed);
}

uint32_t tsc_set_wait_limit(uint32_t sleeps) {
  return g_wait_limit.exchange(sleeps == 0u ? tsc::kDefaultWaitLimit : sleeps,
                               std::memory_order_relaxed);
}

const char* tsc_status_string(int32_t status) {
  switch (status) {
    case TSC_OK: return "TSC_OK";
    case TSC_ERR_INVALID_ARGUMENT: return "TSC_ERR_INVALID_ARGUMENT";
    case TSC_ERR_UNSUPPORTED: return "TSC_ERR_UNSUPPORTED";
    case TSC_ERR_WORKSPACE: return "TSC_ERR_WORKSPACE";
    case TSC_ERR_HIP: return "TSC_ERR_HIP";
    default: return "TSC_UNKNOWN_STATUS";
  }
}

size_t tsc_workspace_size(int64_t B, int64_t V, int64_t R, int32_t W, int32_t dtype) {
  (void)B, (void)V, (void)R, (void)W, (void)dtype;
  return 0;
}

int32_t tsc_sample_with_mask_bits(const void* logits, int32_t dtype, int64_t B, int64_t V,
                                  int64_t ld, const float* temperature, const int32_t* top_k,
                                  const float* top_p, const float* min_p,
                                  const int32_t* optin_rows, int64_t R, const uint64_t* seeds,
                                  const uint64_t* positions, int32_t W, int32_t* tokens,
                                  int8_t* row_status, int32_t* packed_ids, float* logprobs,
                                  int32_t* lengths, float* selected_logprob,
                                  uint8_t* support_bits, int64_t bits_ld, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  (void)workspace;
  if (dtype != TSC_DTYPE_F32 && dtype != TSC_DTYPE_BF16) return TSC_ERR_INVALID_ARGUMENT;
  if (B < 0 || V < 1 || V > INT32_MAX - 16 || ld < V || R < 0 || R > B)
    return TSC_ERR_INVALID_ARGUMENT;
  if (B > 0x7FFFFFFF) return TSC_ERR_UNSUPPORTED;
  if (B == 0) return TSC_OK;
  const size_t esize = dtype == TSC_DTYPE_F32 ? 4 : 2;
  if (!logits || (reinterpret_cast<uintptr_t>(logits) % esize) != 0)
    return TSC_ERR_INVALID_ARGUMENT;
  if (!temperature || !top_k || !top_p || !min_p || !seeds || !positions || !tokens || !row_status)
    return TSC_ERR_INVALID_ARGUMENT;
  if (R > 0) {
    if (!optin_rows || !packed_ids || !lengths || !selected_logprob) return TSC_ERR_INVALID_ARGUMENT;
    if (W < 1) return TSC_ERR_INVALID_ARGUMENT;
    if (W > TSC_MAX_PACKED_WIDTH) return TSC_ERR_UNSUPPORTED;
    if (support_bits != nullptr &&
        (bits_ld < tsc_support_bits_ld(V) || bits_ld % 16 != 0 ||
         (reinterpret_cast<uintptr_t>(support_bits) & 15u) != 0))
      return TSC_ERR_INVALID_ARGUMENT;
  }
  if (workspace_bytes < tsc_workspace_size(B, V, R, W, dtype)) return TSC_ERR_WORKSPACE;

  tsc::SampleArgs a{logits, B, V, ld, temperature, top_k, top_p, min_p, optin_rows, R,
                    seeds, positions, R > 0 ? W : 1, tokens, row_status, packed_ids,
                    logprobs, lengths, selected_logprob,
                    R > 0 ? reinterpret_cast<uint32_t*>(support_bits) : nullptr, bits_ld / 4,
                    g_wait_limit.load(std::memory_order_relaxed)};
  (void)hipGetLastError();  // start from a clean error state so a launch error is ours
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bits = a.bits != nullptr;
  hipError_t err =
      dtype == TSC_DTYPE_F32
          ? (bits ? launch_sampler<TSC_DTYPE_F32, true>(a, s) : launch_sampler<TSC_DTYPE_F32, false>(a, s))
          : (bits ? launch_sampler<TSC_DTYPE_BF16, true>(a, s) : launch_sampler<TSC_DTYPE_BF16, false>(a, s));
  if (err == hipSuccess && R > 0 && g_poison.load(std::memory_order_relaxed) != 0) {
    hipLaunchKernelGGL(tsc::poison_kernel, dim3((unsigned)R), dim3(tsc::kPoisonThreads), 0, s,
                       lengths, packed_ids, logprobs, (int32_t)a.W);
    err = hipGetLastError();
  }
  return err == hipSuccess ? TSC_OK : TSC_ERR_HIP;
}

int32_t tsc_sample_with_mask(const void* logits, int32_t dtype, int64_t B, int64_t V, int64_t ld,
                             const float* temperature, const int32_t* top_k, const float* top_p,
                             const float* min_p, const int32_t* optin_rows, int64_t R,
                             const uint64_t* seeds, const uint64_t* positions, int32_t W,
                             int32_t* tokens, int8_t* row_status, int32_t* packed_ids,
                             float* logprobs, int32_t* lengths, float* selected_logprob,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return tsc_sample_with_mask_bits(logits, dtype, B, V, ld, temperature, top_k, top_p, min_p,
                                   optin_rows, R, seeds, positions, W, tokens, row_status,
                                   packed_ids, logprobs, lengths, selected_logprob, nullptr, 0,
                                   workspace, workspace_bytes, stream);
}

int64_t tsc_support_bits_ld(int64_t V) { return V < 1 ? 0 : tsc::bitmask_words(V) * 4; }

int32_t tsc_support_csr(const int32_t* lengths, const int32_t* packed_ids, const float* logprobs,
                        int64_t R, int32_t W, int64_t* offsets, int32_t* csr_ids,
                        float* csr_logprobs, int64_t cap, void* stream) {
  if (R < 0 || R > 0x7FFFFFFF || cap < 0 || W < 1) return TSC_ERR_INVALID_ARGUMENT;
  if (W > TSC_MAX_PACKED_WIDTH) return TSC_ERR_UNSUPPORTED;
  if (!offsets || (R > 0 && (!lengths || !packed_ids)) || (cap > 0 && !csr_ids))
    return TSC_ERR_INVALID_ARGUMENT;
  tsc::CsrArgs a{lengths, packed_ids, logprobs, R, W, offsets, csr_ids,
                 logprobs ? csr_logprobs : nullptr, cap};
  (void)hipGetLastError();
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (R >= 1 && R <= tsc::kCsrFusedMaxR) {
    hipLaunchKernelGGL(tsc::csr_fused_kernel, dim3((unsigned)R), dim3(tsc::kCsrThreads), 0, s, a);
  } else {
    hipLaunchKernelGGL(tsc::csr_scan_kernel, dim3(1), dim3(tsc::kThreads), 0, s, a);
    if (R > 0)
      hipLaunchKernelGGL(tsc::csr_copy_kernel, dim3((unsigned)R), dim3(tsc::kCsrThreads), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? TSC_OK : TSC_ERR_HIP;
}

int32_t tsc_replay_logprob(const void* logits, int32_t dtype, int64_t N, int64_t V, int64_t ld,
                           const float* temperature, const int32_t* packed_ids,
                           const int32_t* lengths, int32_t W, const int8_t* capture_status,
                           const uint8_t* support_bits, int64_t bits_ld, const int32_t* tokens,
                           float* selected_logprob, float* logprobs, int8_t* row_status,
                           void* stream) {
  if (dtype != TSC_DTYPE_F32 && dtype != TSC_DTYPE_BF16) return TSC_ERR_INVALID_ARGUMENT;
  if (N < 0 || V < 1 || V > INT32_MAX - 16 || ld < V) return TSC_ERR_INVALID_ARGUMENT;
  if (N > 0x7FFFFFFF) return TSC_ERR_UNSUPPORTED;
  if (N == 0) return TSC_OK;
  if (W < 1) return TSC_ERR_INVALID_ARGUMENT;
  if (W > TSC_MAX_PACKED_WIDTH) return TSC_ERR_UNSUPPORTED;
  const size_t esize = dtype == TSC_DTYPE_F32 ? 4 : 2;
  if (!logits || (reinterpret_cast<uintptr_t>(logits) % esize) != 0)
    return TSC_ERR_INVALID_ARGUMENT;
  if (!temperature || !packed_ids || !lengths || !tokens || !selected_logprob || !row_status)
    return TSC_ERR_INVALID_ARGUMENT;
  if (support_bits != nullptr && bits_ld < (V + 7) / 8) return TSC_ERR_INVALID_ARGUMENT;
  tsc::ReplayArgs a{logits, N, V, ld, temperature, packed_ids, lengths, W, capture_status,
                    support_bits, bits_ld, tokens, selected_logprob, logprobs, row_status};
  (void)hipGetLastError();
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  // Support logprobs of bitmask rows read their logits from an LDS stage (bfloat16). That
  // instantiation holds 144 KB of LDS (one workgroup per CU), so it is launched only when a row
  // can be staged at all: V / 8 chunks within the stage's chunk table.
  const bool stage = logprobs != nullptr && support_bits != nullptr && capture_status != nullptr &&
                     (V + 7) / 8 <= (int64_t)tsc::kStageChunks;
  if (dtype == TSC_DTYPE_F32)
    hipLaunchKernelGGL((tsc::replay_kernel<TSC_DTYPE_F32, false>), dim3((unsigned)N), dim3(tsc::kThreads), 0, s, a);
  else if (stage)
    hipLaunchKernelGGL((tsc::replay_kernel<TSC_DTYPE_BF16, true>), dim3((unsigned)N), dim3(tsc::kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((tsc::replay_kernel<TSC_DTYPE_BF16, false>), dim3((unsigned)N), dim3(tsc::kThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? TSC_OK : TSC_ERR_HIP;
}

}  // extern "C"
