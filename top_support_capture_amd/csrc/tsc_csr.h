// Compressed (CSR) layout of captured supports: the packed [R, W] capture written back to back,
// so that a copy to the host can be sized by the realized support instead of R * W (sglang PR
// #40986, "Limitations": the packed buffer crosses whole, sized by its capacity).
//
// Up to kCsrFusedMaxR slots, one launch: workgroup j sums the clamped lengths of the slots before
// it itself (at most kCsrFusedMaxR reads, served by L2 after the first workgroups), writes
// offsets[j + 1], and copies its first lengths[j] ids (and logprobs) to offsets[j] ..
// offsets[j + 1] with coalesced loads and stores. More slots take two launches: one workgroup
// scans the R lengths into offsets[0..R], then the same copy per slot.
#pragma once

#include "tsc_device.h"

namespace tsc {

struct CsrArgs {
  const int32_t* lengths;     // [R]
  const int32_t* packed_ids;  // [R, W]
  const float* logprobs;      // [R, W] or null
  int64_t R;
  int32_t W;
  int64_t* offsets;   // [R + 1]
  int32_t* ids;       // [cap]
  float* lps;         // [cap] or null
  int64_t cap;
};

__device__ inline int64_t csr_len(int32_t n, int32_t W) { return n < 0 ? 0 : (n > W ? W : n); }

// offsets[0] = 0, offsets[j + 1] = offsets[j] + clamp(lengths[j], 0, W): chunks of 1024 lengths,
// a wave scan plus a scan of the wave totals, carried from chunk to chunk.
__global__ void __launch_bounds__(kThreads) csr_scan_kernel(CsrArgs a) {
  __shared__ int64_t wave_tot[kWaves];
  const uint32_t tid = threadIdx.x, lane = tid & (kWaveSize - 1), w = tid / kWaveSize;
  int64_t carry = 0;
  if (tid == 0) a.offsets[0] = 0;
  for (int64_t base = 0; base < a.R; base += kThreads) {
    const int64_t j = base + tid;
    const int64_t v = j < a.R ? csr_len(a.lengths[j], a.W) : 0;
    const int64_t incl = wave_incl_scan(v, SumOp(), (int64_t)0);
    if (lane == kWaveSize - 1) wave_tot[w] = incl;
    lds_barrier();
    int64_t total;
    const int64_t before = waves_prefix(wave_tot, SumOp(), (int64_t)0, total);
    if (j < a.R) a.offsets[j + 1] = carry + before + incl;
    carry += total;
    lds_barrier();  // wave_tot is rewritten by the next chunk
  }
}

constexpr int kCsrThreads = 256;
constexpr int64_t kCsrFusedMaxR = 2048;

// Slot j's prefix to offset `at`; entries at or past cap are not written. A thread moves kU
// entries per step, all their loads before any store, so that a long prefix costs a few round
// trips rather than one per entry.
// The copy loop, with nontemporal stores or ordinary ones (separate instantiations: a run-time
// choice between two otherwise equal stores is merged by the compiler into one ordinary store).
template <bool NT>
__device__ inline void csr_copy_run(const CsrArgs& a, const int32_t* src, const float* srcl,
                                    int64_t at, int64_t lim) {
  constexpr int kU = 8;
  for (int64_t i0 = threadIdx.x; i0 < lim; i0 += (int64_t)kCsrThreads * kU) {
    int32_t v[kU];
    float l[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + (int64_t)u * kCsrThreads;
      v[u] = i < lim ? src[i] : 0;
      l[u] = srcl && i < lim ? srcl[i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t i = i0 + (int64_t)u * kCsrThreads;
      if (i < lim) {
        if constexpr (NT) {
          __builtin_nontemporal_store(v[u], &a.ids[at + i]);
          if (srcl) __builtin_nontemporal_store(l[u], &a.lps[at + i]);
        } else {
          a.ids[at + i] = v[u];
          if (srcl) a.lps[at + i] = l[u];
        }
      }
    }
  }
}

__device__ inline void csr_copy_slot(const CsrArgs& a, int64_t j, int64_t n, int64_t at) {
  const int32_t* src = a.packed_ids + j * a.W;
  const float* srcl = a.logprobs && a.lps ? a.logprobs + j * a.W : nullptr;
  const int64_t room = a.cap - at;
  const int64_t lim = n < room ? n : (room > 0 ? room : 0);
  // Long slots are written with nontemporal stores: they stream to memory as they are written
  // instead of staying dirty in L2 for the kernel's end to write back (the 2M entries of a B=256
  // capture at width 8192: 6.5 -> 5.5 us). Short slots keep ordinary stores: their partial lines
  // at both ends made the CSR of a B=256, V=151936 capture (about 1100 entries a slot) slower,
  // 3.4 -> 4.1 us.
  if (lim >= (int64_t)kNtStoreMin)
    csr_copy_run<true>(a, src, srcl, at, lim);
  else
    csr_copy_run<false>(a, src, srcl, at, lim);
}

// Workgroup j copies slot j's prefix to the offset the scan wrote.
__global__ void __launch_bounds__(kCsrThreads) csr_copy_kernel(CsrArgs a) {
  const int64_t j = blockIdx.x;
  csr_copy_slot(a, j, csr_len(a.lengths[j], a.W), a.offsets[j]);
}

// Workgroup j (R <= kCsrFusedMaxR): its offset from the lengths before it, then its copy.
__global__ void __launch_bounds__(kCsrThreads) csr_fused_kernel(CsrArgs a) {
  constexpr int kW = kCsrThreads / kWaveSize;
  __shared__ int64_t part[kW];
  const int64_t j = blockIdx.x;
  const uint32_t tid = threadIdx.x;
  int64_t s = 0;
  for (int64_t i = tid; i < j; i += kCsrThreads) s += csr_len(a.lengths[i], a.W);
  s = wave_reduce(s, SumOp());
  if ((tid & (kWaveSize - 1)) == 0) part[tid / kWaveSize] = s;
  lds_barrier();
  int64_t at = 0;
#pragma unroll
  for (int i = 0; i < kW; ++i) at += part[i];
  const int64_t n = csr_len(a.lengths[j], a.W);
  if (tid == 0) {
    if (j == 0) a.offsets[0] = 0;
    a.offsets[j + 1] = at + n;
  }
  csr_copy_slot(a, j, n, at);
}

// Slot r's packed entries past its length (clamped to [0, W]) become id -1 and logprob NaN: a
// debugging aid (tsc_set_debug_poison) that makes reads past a capture's length visible.
constexpr int kPoisonThreads = 256;
__global__ void __launch_bounds__(kPoisonThreads) poison_kernel(const int32_t* lengths,
                                                                int32_t* packed_ids,
                                                                float* logprobs, int32_t W) {
  const int64_t r = blockIdx.x;
  const int32_t l = lengths[r];
  const int32_t from = l < 0 ? 0 : (l > W ? W : l);
  for (int32_t j = from + (int32_t)threadIdx.x; j < W; j += kPoisonThreads) {
    packed_ids[r * W + j] = -1;
    if (logprobs) logprobs[r * W + j] = __builtin_nanf("");
  }
}

}  // namespace tsc
