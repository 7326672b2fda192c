// Replay of a captured support under new logits: the log-softmax of the row restricted to the
// support, at the sampled token (vLLM "Sampling Mask / Distribution Replay" article, section
// "RL training side: computing pi_theta with the mask": the training model's logits are masked
// to the support the sampler returned, so that pi_theta and pi_old share one normalizer).
//
// One workgroup per row. The support is either the row's packed ids (a gather of at most W
// logits) or, for a row whose capture overflowed, its bitmask (a pass over ceil(V / 8) mask
// bytes that loads only the logits of set bits). Each thread keeps an online maximum and sum of
// exp((x - max) / T) over its share; one block reduction of the maxima, one of the rescaled
// sums, then the token's logprob in float64.
#pragma once

#include "tsc_device.h"

namespace tsc {

struct ReplayArgs {
  const void* logits;
  int64_t N, V, ld;
  const float* temperature;
  const int32_t* packed_ids;  // [N, W]
  const int32_t* lengths;     // [N]
  int32_t W;
  const int8_t* capture_status;  // [N] or null
  const uint8_t* bits;           // [N, bits_ld] or null
  int64_t bits_ld;               // bytes
  const int32_t* tokens;         // [N]
  float* selected_logprob;       // [N]
  float* logprobs;               // [N, W] or null
  int8_t* row_status;            // [N]
};

struct ReplayShared {
  uint64_t red[kWaves];
};

// Online log-sum-exp state of one thread: m the largest finite logit seen, s = sum of
// exp2((x - m) * c) over the finite ones (c = log2(e) / T).
struct OnlineLse {
  float m = -__builtin_inff();
  float s = 0.0f;
  uint32_t bad = 0;  // a NaN or +inf logit
  uint32_t n = 0;    // support entries seen
  __device__ inline void add(float x, float c) {
    ++n;
    if (x != x || x == __builtin_inff()) {
      bad = 1;
    } else if (x > m) {
      s = s * __builtin_amdgcn_exp2f((m - x) * c) + 1.0f;  // m = -inf: s is 0, 0 * 0 + 1
      m = x;
    } else if (x != -__builtin_inff()) {
      s += __builtin_amdgcn_exp2f((x - m) * c);
    }
  }
};

template <int DT>
__global__ void __launch_bounds__(kThreads) replay_kernel(ReplayArgs a) {
  using E = Elem<DT>;
  __shared__ ReplayShared sh;
  const int64_t j = blockIdx.x;
  const uint32_t tid = threadIdx.x;
  const auto* row = reinterpret_cast<const typename E::Bits*>(a.logits) + j * a.ld;
  const int64_t V = a.V;

  const int32_t cs = a.capture_status ? (int32_t)a.capture_status[j] : TSC_ROW_OK;
  if (cs >= TSC_ROW_NO_SUPPORT) {  // nothing was captured for this row
    if (tid == 0) {
      a.row_status[j] = (int8_t)cs;
      a.selected_logprob[j] = __builtin_nanf("");
    }
    return;
  }
  const float T = a.temperature[j];
  const int32_t n = a.lengths[j];
  const int32_t tok = a.tokens[j];
  const bool from_bits = cs == TSC_ROW_OVERFLOW;
  const bool n_ok = n >= 1 && n <= a.W;
  bool ok = __builtin_isfinite(T) && T >= 1.1754943508222875e-38f && tok >= 0 && tok < V &&
            (from_bits ? a.bits != nullptr : n_ok);
  if (!ok) {
    if (tid == 0) {
      a.row_status[j] = TSC_ROW_INVALID_PARAM;
      a.selected_logprob[j] = __builtin_nanf("");
    }
    return;
  }
  const float c = 1.4426950408889634f / T;
  OnlineLse acc;
  uint32_t bad_id = 0, found = 0;
  const int32_t* ids = a.packed_ids + j * a.W;
  if (!from_bits) {
    for (int32_t i = (int32_t)tid; i < n; i += kThreads) {
      const int32_t id = ids[i];
      if (id < 0 || id >= V) {
        bad_id = 1;
        continue;
      }
      found |= id == tok;
      acc.add(E::to_float((uint32_t)row[id]), c);
    }
  } else {
    // Chunks of 8 ids, one mask byte each; neighbouring lanes take neighbouring chunks.
    const uint8_t* brow = a.bits + j * a.bits_ld;
    const int64_t nchunks = (V + 7) / 8;
    for (int64_t ch = tid; ch < nchunks; ch += kThreads) {
      uint32_t byte = brow[ch];
      if (ch == nchunks - 1 && (V & 7)) byte &= (1u << (V & 7)) - 1u;  // bits past V
      if (byte == 0u) continue;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        x[e] = (byte >> e) & 1u ? E::to_float((uint32_t)row[ch * 8 + e]) : -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((byte >> e) & 1u) acc.add(x[e], c);
      if ((int64_t)tok >> 3 == ch) found |= (byte >> (tok & 7)) & 1u;
    }
  }
  // Block reductions: the maximum, then the sums rescaled to it, and the flags.
  const float M = block_reduce(acc.m, MaxOp(), sh.red);
  const float sr = acc.m == -__builtin_inff() ? 0.0f : acc.s * __builtin_amdgcn_exp2f((acc.m - M) * c);
  const float S = block_reduce(sr, SumOp(), sh.red);
  const uint32_t flags = block_reduce((acc.bad ? 1u : 0u) | (bad_id ? 2u : 0u) | (found ? 4u : 0u) |
                                          (acc.n ? 8u : 0u),
                                      [](uint32_t x, uint32_t y) { return x | y; }, sh.red);
  int8_t status = TSC_ROW_OK;
  if ((flags & 2u) || !(flags & 8u)) status = TSC_ROW_INVALID_PARAM;  // bad id, empty support
  else if (flags & 1u) status = TSC_ROW_NONFINITE;
  else if (M == -__builtin_inff()) status = TSC_ROW_NO_SUPPORT;
  const double lnS = log((double)S);
  if (tid == 0) {
    a.row_status[j] = status;
    float sel = __builtin_nanf("");
    if (status == TSC_ROW_OK) {
      const float xt = E::to_float((uint32_t)row[tok]);
      sel = (flags & 4u) ? (float)(((double)xt - (double)M) / (double)T - lnS) : -__builtin_inff();
    }
    a.selected_logprob[j] = sel;
  }
  // The logprob of every packed entry (for an overflowing row, of its packed prefix).
  if (a.logprobs != nullptr && status == TSC_ROW_OK && n_ok) {
    float* out = a.logprobs + j * a.W;
    const uint8_t* brow = from_bits ? a.bits + j * a.bits_ld : nullptr;
    for (int32_t i = (int32_t)tid; i < n; i += kThreads) {
      const int32_t id = ids[i];
      // Masked log-softmax: an id outside the support (possible only in a bitmask row) is -inf.
      const bool in = id >= 0 && id < V && (brow == nullptr || ((brow[id >> 3] >> (id & 7)) & 1u));
      const float x = in ? E::to_float((uint32_t)row[id]) : -__builtin_inff();
      out[i] = (float)(((double)x - (double)M) / (double)T - lnS);
    }
  }
}

}  // namespace tsc
