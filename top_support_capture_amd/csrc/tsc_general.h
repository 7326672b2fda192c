// General sampler kernel: one 1024-thread workgroup per row, several passes over the row.
//
// It serves every row the library accepts (any dtype, any V, every filter combination,
// supports wider than on-chip storage) and is the reference GPU path. Per row, in order:
//   1. stats pass: maximum key (and its first index), finite count, NaN/+inf detection;
//   2. mass pass (only when top_p < 1): Z = sum of fixed-point weights over finite tokens;
//   3. radix descent for the joint top-k/top-p threshold: per 8-bit digit one pass builds count
//      (and mass) histograms of the keys under the current prefix, and one wavefront picks the
//      lowest digit that still satisfies "fewer than k tokens above" and "mass above <= top_p*Z";
//   4. survivor pass: support size L, support mass, and the exponential race in float64;
//   5. opt-in rows only: the first min(L, W) support entries in (logit desc, id asc) order are
//      gathered into LDS (a second descent picks the W-th key, and a descent on ids the tied
//      cut, when L exceeds the LDS capacity), bitonic-sorted and written with their logprobs.
#pragma once

#include "tsc_device.h"

namespace tsc {

struct SampleArgs {
  const void* logits;
  int64_t B, V, ld;
  const float* temperature;
  const int32_t* top_k;
  const float* top_p;
  const float* min_p;
  const int32_t* optin_rows;
  int64_t R;
  const uint64_t* seeds;
  const uint64_t* positions;
  int32_t W;
  int32_t* tokens;
  int8_t* row_status;
  int32_t* packed_ids;
  float* logprobs;
  int32_t* lengths;
  float* selected_logprob;
  uint32_t* bits;   // [R, bits_ld] support bitmasks of OVERFLOW slots, or null
  int64_t bits_ld;  // row stride of `bits` in 32-bit words (a multiple of 4)
  uint32_t wait_limit;  // sleeps a wait between the waves of a workgroup may take (>= 1)
};

// Words of a support bitmask row that a kernel writes: the bits of ids 0..V-1 (bit i in word
// i / 32 at position i % 32, the little-endian bit order of a byte array), zero-padded to a whole
// number of 16-byte units.
__host__ __device__ inline int64_t bitmask_words(int64_t V) { return (V + 127) / 128 * 4; }

constexpr int kSortCap = TSC_MAX_PACKED_WIDTH;                 // u64 entries in the LDS buffer
constexpr size_t kGeneralDynLds = (size_t)kSortCap * sizeof(uint64_t);

// Calls f(id, bits) for every element of the row handled by this thread, 16-byte loads when the
// row is 16-byte aligned, scalar loads otherwise and for the tail.
template <class E, class F>
__device__ inline void visit_row(const typename E::Bits* row, int64_t V, F&& f) {
  int64_t done = 0;
  if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0) {
    const uint4* v = reinterpret_cast<const uint4*>(row);
    const int64_t nv = V / E::kVec;
    auto visit16 = [&](const uint4& d, int64_t i) {
      const uint32_t w[4] = {d.x, d.y, d.z, d.w};
      const int32_t base = (int32_t)(i * E::kVec);
      if constexpr (E::kVec == 8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          f(base + 2 * j, w[j] & 0xFFFFu);
          f(base + 2 * j + 1, w[j] >> 16);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) f(base + j, w[j]);
      }
    };
    // Two loads per thread in flight before either is used (their latencies overlap), then the
    // remainder one at a time.
    constexpr int kU = 2;
    int64_t i = threadIdx.x;
    for (; i + (kU - 1) * kThreads < nv; i += kU * kThreads) {
      uint4 d[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) d[u] = v[i + u * kThreads];
#pragma unroll
      for (int u = 0; u < kU; ++u) visit16(d[u], i + u * kThreads);
    }
    for (; i < nv; i += kThreads) visit16(v[i], i);
    done = nv * E::kVec;
  }
  for (int64_t i = done + threadIdx.x; i < V; i += kThreads) f((int32_t)i, (uint32_t)row[i]);
}

struct DescentState {
  uint32_t prefix;   // resolved high digits of the answer
  uint32_t above;    // elements (under the predicate) with a value above the current range
  uint64_t mabove;   // their fixed-point mass
};

struct GeneralShared {
  uint32_t cnt[256];
  uint64_t mass[256];
  uint64_t red[kWaves];
  uint32_t pick_digit;
  uint32_t pick_above;
  uint64_t pick_mabove;
  uint32_t nbuf;
};

// Radix descent over NBITS-bit values val(id, bits) of the elements that satisfy pred(id, bits):
// finds the smallest present value v with #(values > v) < kk and, when use_mass, mass(> v) <= pz,
// where mass sums wfix(bits). Requires at least one element and kk >= 1, pz >= 0.
template <class E, int NBITS, class Pred, class Val, class Mass>
__device__ __forceinline__ DescentState radix_descent(const typename E::Bits* row, int64_t V, Pred pred, Val val,
                                      uint32_t kk, bool use_mass, double pz, Mass wfix,
                                      GeneralShared& sh) {
  DescentState st{0u, 0u, 0ull};
  const int lane = threadIdx.x & (kWaveSize - 1);
  for (int shift = NBITS - 8; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += kThreads) {
      sh.cnt[i] = 0u;
      sh.mass[i] = 0ull;
    }
    __syncthreads();
    const uint32_t hi_mask = (shift + 8 >= 32) ? 0u : (0xFFFFFFFFu << (shift + 8));
    const uint32_t want = st.prefix & hi_mask;
    visit_row<E>(row, V, [&](int32_t id, uint32_t b) {
      if (!pred(id, b)) return;
      const uint32_t v = val(id, b);
      if ((v & hi_mask) != want) return;
      const uint32_t d = (v >> shift) & 255u;
      atomicAdd(&sh.cnt[d], 1u);
      if (use_mass) atomicAdd((unsigned long long*)&sh.mass[d], (unsigned long long)wfix(b));
    });
    __syncthreads();
    if (threadIdx.x < kWaveSize) {
      // Lane l owns digits 4l..4l+3. Suffix sums run from the highest digit down.
      uint32_t c[4];
      uint64_t m[4];
      uint32_t ct = 0;
      uint64_t mt = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = sh.cnt[4 * lane + q];
        m[q] = sh.mass[4 * lane + q];
        ct += c[q];
        mt += m[q];
      }
      uint32_t cs = ct;
      uint64_t ms = mt;
#pragma unroll
      for (int o = 1; o < kWaveSize; o <<= 1) {
        const uint32_t tc = __shfl_down(cs, o, kWaveSize);
        const uint64_t tm = __shfl_down(ms, o, kWaveSize);
        if (lane + o < kWaveSize) {
          cs += tc;
          ms += tm;
        }
      }
      uint32_t g = st.above + (cs - ct);  // elements above this lane's highest digit
      uint64_t mg = st.mabove + (ms - mt);
      uint32_t best = 256u, bg = 0u;
      uint64_t bm = 0ull;
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        const bool ok = c[q] > 0u && g < kk && (!use_mass || (double)mg <= pz);
        if (ok) {
          best = 4u * lane + q;
          bg = g;
          bm = mg;
        }
        g += c[q];
        mg += m[q];
      }
      const uint32_t lowest = wave_reduce(best, MinOp());
      if (best == lowest && lowest < 256u) {
        sh.pick_digit = lowest;
        sh.pick_above = bg;
        sh.pick_mabove = bm;
      }
    }
    __syncthreads();
    st.prefix |= sh.pick_digit << shift;
    st.above = sh.pick_above;
    st.mabove = sh.pick_mabove;
    __syncthreads();
  }
  return st;
}

// Logprob of a support entry with logit x: (x - m) / T - ln Z_S, in float64, rounded once.
// Contraction is off so that the packed entry and the selected logprob are bit-identical.
__device__ inline float logprob_of(float x, float m, float T, double lnzs) {
#pragma clang fp contract(off)
  const double s = ((double)x - (double)m) / (double)T;
  return (float)(s - lnzs);
}

// Capture slot of row b (-1 if it has none) under the slot-validity rule: slot j is valid iff
// 0 <= optin_rows[j] < B and it exceeds every earlier entry. The workgroup of row b also owns slot
// b's validity and marks it (length 0, NaN selected logprob) when it is invalid.
__device__ inline int64_t find_capture_slot(const SampleArgs& a, int64_t b, uint64_t* red) {
  const int tid = threadIdx.x;
  int32_t my_slot = -1;
  bool slot_b_invalid = false;
  int32_t carry = INT32_MIN;
  for (int64_t base = 0; base < a.R; base += kThreads) {
    const int64_t j = base + tid;
    const int32_t e = j < a.R ? a.optin_rows[j] : INT32_MIN;
    // Inclusive max-scan over the chunk: wave scan, then wave totals.
    int32_t inc = e;
    const int lane = tid & (kWaveSize - 1);
#pragma unroll
    for (int o = 1; o < kWaveSize; o <<= 1) {
      const int32_t t = __shfl_up(inc, o, kWaveSize);
      if (lane >= o) inc = inc > t ? inc : t;
    }
    int32_t* wt = reinterpret_cast<int32_t*>(red);
    lds_barrier();
    if (lane == kWaveSize - 1) wt[tid / kWaveSize] = inc;
    lds_barrier();
    int32_t all;
    const int32_t wbefore = waves_prefix(wt, MaxOp(), INT32_MIN, all);
    const int32_t before = carry > wbefore ? carry : wbefore;
    int32_t excl = __shfl_up(inc, 1, kWaveSize);
    if (lane == 0) excl = INT32_MIN;
    excl = excl > before ? excl : before;
    const int32_t chunk_max = carry > all ? carry : all;
    if (j < a.R) {
      const bool valid = e >= 0 && (int64_t)e < a.B && e > excl;
      if (valid && (int64_t)e == b) my_slot = (int32_t)j;
      if (!valid && j == b) slot_b_invalid = true;
    }
    carry = chunk_max;
  }
  my_slot = block_reduce(my_slot, MaxOp(), red);
  if (slot_b_invalid) {
    a.lengths[b] = 0;
    a.selected_logprob[b] = __builtin_nanf("");
  }
  return my_slot;
}

// Writes the outputs of a row that has no support (status >= 2): token -1, empty capture.
__device__ inline void finish_empty_row(const SampleArgs& a, int64_t b, int64_t slot, int8_t status) {
  if (threadIdx.x == 0) {
    a.tokens[b] = -1;
    a.row_status[b] = status;
    if (slot >= 0) {
      a.lengths[slot] = 0;
      a.selected_logprob[slot] = __builtin_nanf("");
    }
  }
}

// Temperature 0 or a normal positive finite float; top_p and min_p in [0, 1] (false for NaN).
__device__ inline bool row_params_valid(float T, float p, float mp) {
  const bool t_ok = __builtin_isfinite(T) && T >= 0.0f && (T == 0.0f || T >= 1.1754943508222875e-38f);
  return t_ok && p >= 0.0f && p <= 1.0f && mp >= 0.0f && mp <= 1.0f;
}

// The whole sampling of row b by the general multi-pass algorithm. `sortbuf` holds kSortCap
// u64 entries of LDS. Every thread of the workgroup calls it; it returns with the row done.
template <int DT, bool BITS>
__device__ __forceinline__ void general_row(const SampleArgs& a, int64_t b, int64_t slot, uint64_t* sortbuf,
                            GeneralShared& sh) {
  using E = Elem<DT>;
  const int tid = threadIdx.x;
  const auto* row = reinterpret_cast<const typename E::Bits*>(a.logits) + b * a.ld;
  const int64_t V = a.V;

  // ---- Parameters ---------------------------------------------------------------------------
  const float T = a.temperature[b];
  const int32_t k = a.top_k[b];
  const float p = a.top_p[b];
  const float mp = a.min_p[b];
  if (!row_params_valid(T, p, mp)) {
    finish_empty_row(a, b, slot, TSC_ROW_INVALID_PARAM);
    return;
  }
  // ---- 1. Stats pass ------------------------------------------------------------------------
  uint64_t best_packed = 0;  // (key << 32) | (0x7FFFFFFF - id): max = largest key, first id
  uint32_t nfin = 0, bad = 0, kmin = 0xFFFFFFFFu;
  visit_row<E>(row, V, [&](int32_t id, uint32_t bits) {
    if (is_finite_bits<E>(bits)) {
      const uint32_t kk = key_of<E>(bits);
      const uint64_t pk = ((uint64_t)kk << 32) | (uint32_t)(0x7FFFFFFF - id);
      best_packed = pk > best_packed ? pk : best_packed;
      kmin = kk < kmin ? kk : kmin;
      ++nfin;
    } else if (bits != E::kNegInf) {
      bad = 1;
    }
  });
  best_packed = block_reduce(best_packed, MaxOp(), sh.red);
  nfin = block_reduce(nfin, SumOp(), sh.red);
  bad = block_reduce(bad, MaxOp(), sh.red);
  kmin = block_reduce(kmin, MinOp(), sh.red);
  if (bad) {
    finish_empty_row(a, b, slot, TSC_ROW_NONFINITE);
    return;
  }
  if (nfin == 0) {
    finish_empty_row(a, b, slot, TSC_ROW_NO_SUPPORT);
    return;
  }
  const uint32_t kmax = (uint32_t)(best_packed >> 32);
  const int32_t argmax = 0x7FFFFFFF - (int32_t)(uint32_t)best_packed;
  const float m = E::to_float(bits_of_key<E>(kmax));

  if (T == 0.0f) {  // greedy: width-1 support, logprob 0
    if (tid == 0) {
      a.tokens[b] = argmax;
      a.row_status[b] = TSC_ROW_OK;
      if (slot >= 0) {
        a.packed_ids[slot * a.W] = argmax;
        if (a.logprobs) a.logprobs[slot * a.W] = 0.0f;
        a.lengths[slot] = 1;
        a.selected_logprob[slot] = 0.0f;
      }
    }
    return;
  }

  const uint32_t k_eff = (k >= 1 && (uint32_t)k < nfin) ? (uint32_t)k : nfin;
  const bool need_p = p < 1.0f;
  const bool need_m = mp > 0.0f;
  const float c = 1.4426950408889634f / T;  // log2(e) / T
  // Fixed-point weight 2^fx * exp((x - m) / T) with fx = 62 - bitlength(V), so a row's total
  // stays below 2^62: integer sums are exact, so every histogram and the total agree bit for
  // bit whatever the summation order.
  const double fx_scale = __builtin_ldexp(1.0, 62 - (32 - __builtin_clz((uint32_t)V)));
  auto wfix = [&](uint32_t bits) -> uint64_t {
    const float w = __builtin_amdgcn_exp2f((E::to_float(bits) - m) * c);
    return (uint64_t)((double)w * fx_scale);
  };
  auto finite_pred = [&](int32_t, uint32_t bits) { return is_finite_bits<E>(bits); };
  auto key_val = [&](int32_t, uint32_t bits) { return key_of<E>(bits); };

  // ---- 2. Total mass (top-p only) -------------------------------------------------------------
  double pz = 0.0;
  if (need_p) {
    uint64_t z = 0;
    visit_row<E>(row, V, [&](int32_t, uint32_t bits) {
      if (is_finite_bits<E>(bits)) z += wfix(bits);
    });
    z = block_reduce(z, SumOp(), sh.red);
    pz = (double)p * (double)z;
  }

  // ---- 3. Joint top-k / top-p threshold -------------------------------------------------------
  uint32_t tkp;
  if (!need_p && k_eff == nfin) {
    tkp = kmin;
  } else {
    tkp = radix_descent<E, E::kKeyBits>(row, V, finite_pred, key_val, k_eff, need_p, pz, wfix, sh)
              .prefix;
  }
  const double ln_mp = need_m ? log((double)mp) : 0.0;
  auto surv = [&](int32_t, uint32_t bits) {
    if (!is_finite_bits<E>(bits)) return false;
    if (key_of<E>(bits) < tkp) return false;
    if (!need_m) return true;
    return ((double)E::to_float(bits) - (double)m) / (double)T >= ln_mp;
  };

  // ---- 4. Survivors: size, mass, race -----------------------------------------------------------
  const uint64_t seed = a.seeds[b], pos = a.positions[b];
  uint32_t L = 0;
  double zs = 0.0, best_score = -__builtin_inf();
  int32_t best_id = 0x7FFFFFFF;
  visit_row<E>(row, V, [&](int32_t id, uint32_t bits) {
    if (!surv(id, bits)) return;
    ++L;
    const double s = ((double)E::to_float(bits) - (double)m) / (double)T;
    zs += exp(s);
    const double u = race_uniform((uint32_t)id, seed, pos);
    const double score = s - log(-log(u));
    if (score > best_score || (score == best_score && id < best_id)) {
      best_score = score;
      best_id = id;
    }
  });
  L = block_reduce(L, SumOp(), sh.red);
  zs = block_reduce(zs, SumOp(), sh.red);
  const double top = block_reduce(best_score, MaxOp(), sh.red);
  const int32_t token = block_reduce(best_score == top ? best_id : 0x7FFFFFFF, MinOp(), sh.red);
  const double lnzs = log(zs);

  if (tid == 0) {
    a.tokens[b] = token;
    a.row_status[b] = (slot >= 0 && L > (uint32_t)a.W) ? TSC_ROW_OVERFLOW : TSC_ROW_OK;
  }
  if (slot < 0) return;

  // ---- 5. Ordered capture ---------------------------------------------------------------------
  const uint32_t W = (uint32_t)a.W;
  if (BITS && a.bits != nullptr && L > W) {
    // The exact support of a row wider than W, as a bitmask: each thread builds whole words.
    uint32_t* brow = a.bits + slot * a.bits_ld;
    const int64_t nw = bitmask_words(V);
    for (int64_t j = tid; j < nw; j += kThreads) {
      uint32_t word = 0;
      const int64_t i0 = j * 32;
      const int n = i0 >= V ? 0 : (V - i0 < 32 ? (int)(V - i0) : 32);
      for (int e = 0; e < n; ++e)
        word |= (uint32_t)surv((int32_t)(i0 + e), (uint32_t)row[i0 + e]) << e;
      brow[j] = word;
    }
  }
  const uint32_t len = L < W ? L : W;
  // Gather predicate: everything when the support fits the LDS buffer, else the first W in
  // order: keys above the W-th key, plus the lowest ids of its tie group.
  uint32_t t_w = tkp, id_cut = 0x7FFFFFFFu;
  bool cut_ids = false;
  if (L > (uint32_t)kSortCap) {
    const DescentState d = radix_descent<E, E::kKeyBits>(row, V, surv, key_val, W, false, 0.0,
                                                         wfix, sh);
    t_w = d.prefix;
    const uint32_t n_gt = d.above;
    uint32_t tied = 0;
    visit_row<E>(row, V, [&](int32_t id, uint32_t bits) {
      if (surv(id, bits) && key_of<E>(bits) == t_w) ++tied;
    });
    tied = block_reduce(tied, SumOp(), sh.red);
    if (n_gt + tied > (uint32_t)kSortCap) {
      cut_ids = true;
      auto tied_pred = [&](int32_t id, uint32_t bits) {
        return surv(id, bits) && key_of<E>(bits) == t_w;
      };
      auto inv_id = [&](int32_t id, uint32_t) { return ~(uint32_t)id; };
      id_cut = ~radix_descent<E, 32>(row, V, tied_pred, inv_id, W - n_gt, false, 0.0, wfix, sh)
                    .prefix;
    }
  }
  if (tid == 0) sh.nbuf = 0;
  __syncthreads();
  visit_row<E>(row, V, [&](int32_t id, uint32_t bits) {
    if (!surv(id, bits)) return;
    const uint32_t kk = key_of<E>(bits);
    if (kk < t_w) return;
    if (cut_ids && kk == t_w && (uint32_t)id > id_cut) return;
    const uint32_t at = atomicAdd(&sh.nbuf, 1u);
    sortbuf[at] = ((uint64_t)(~kk & E::kMask) << 32) | (uint32_t)id;
  });
  __syncthreads();
  const uint32_t n = sh.nbuf;
  uint32_t n2 = 1;
  while (n2 < n) n2 <<= 1;
  for (uint32_t i = n + tid; i < n2; i += kThreads) sortbuf[i] = ~0ull;
  __syncthreads();
  for (uint32_t kk = 2; kk <= n2; kk <<= 1) {
    for (uint32_t j = kk >> 1; j > 0; j >>= 1) {
      for (uint32_t i = tid; i < n2; i += kThreads) {
        const uint32_t ixj = i ^ j;
        if (ixj > i) {
          const uint64_t x = sortbuf[i], y = sortbuf[ixj];
          const bool up = (i & kk) == 0;
          if ((x > y) == up) {
            sortbuf[i] = y;
            sortbuf[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  int32_t* out_ids = a.packed_ids + slot * a.W;
  float* out_lp = a.logprobs ? a.logprobs + slot * a.W : nullptr;
  for (uint32_t j = tid; j < len; j += kThreads) {
    const uint64_t e = sortbuf[j];
    out_ids[j] = (int32_t)(uint32_t)e;
    if (out_lp) {
      const uint32_t kk = ~(uint32_t)(e >> 32) & E::kMask;
      out_lp[j] = logprob_of(E::to_float(bits_of_key<E>(kk)), m, T, lnzs);
    }
  }
  if (tid == 0) {
    a.lengths[slot] = (int32_t)len;
    a.selected_logprob[slot] = logprob_of(E::to_float((uint32_t)row[token]), m, T, lnzs);
  }
}

template <int DT>
__global__ void __launch_bounds__(kThreads) sample_general_kernel(SampleArgs a) {
  extern __shared__ uint64_t sortbuf[];
  __shared__ GeneralShared sh;
  const int64_t b = blockIdx.x;
  const int64_t slot = find_capture_slot(a, b, sh.red);
  general_row<DT, true>(a, b, slot, sortbuf, sh);
}

}  // namespace tsc
