// Greedy rows (temperature 0) in one read: the first index of the row maximum.
//
// A greedy row's support is that one token, with logprob 0 (temperature 0 as the limit of the
// softmax: the whole mass on the maximum; the first index breaks ties, as an argmax does). A NaN
// or +inf logit makes the row NONFINITE, a row of -inf only NO_SUPPORT, as for sampled rows.
//
// Every thread streams 16-byte loads, eight in flight, and keeps two maxima of its values: one
// with ordinary comparisons (NaN never wins one), with the first of its loads that reached it,
// and one with the NaN-propagating maximum, whose NaN or +inf marks the row nonfinite. After a
// block reduction only the threads whose maximum equals the row maximum read their recorded load
// again and report its first element equal to the maximum (-0 equals +0); the smallest reported
// id is the token.
#pragma once

namespace tsc {

constexpr int kGreedyInFlight = 8;  // 16-byte loads in flight per thread
constexpr int64_t kGreedyMaxV = (int64_t)1 << 26;  // byte offsets within a row fit 32 bits

// Rows this pass serves: temperature 0 with valid parameters, 16-byte aligned rows.
template <int DT>
__device__ inline bool greedy_eligible(const SampleArgs& a, float T, float p, float mp) {
  constexpr int64_t kVec = Elem<DT>::kVec;
  return T == 0.0f && row_params_valid(T, p, mp) && a.V <= kGreedyMaxV && a.ld % kVec == 0 &&
         (reinterpret_cast<uintptr_t>(a.logits) & 15u) == 0;
}

template <int DT>
__device__ __forceinline__ void greedy_row(const SampleArgs& a, int64_t b, int64_t slot,
                                           uint64_t* red) {
  using E = Elem<DT>;
  constexpr int kVec = E::kVec;
  constexpr uint32_t kNegInf4 = DT == TSC_DTYPE_BF16 ? 0xFF80FF80u : 0xFF800000u;
  const uint32_t tid = threadIdx.x;
  const auto* row = reinterpret_cast<const typename E::Bits*>(a.logits) + b * a.ld;
  const uint32_t nv = (uint32_t)(a.V / kVec);  // whole 16-byte chunks (the row is 16-byte aligned)
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<typename E::Bits*>(row), (short)0, (int)(nv * 16u), 0x00020000);

  auto unpack = [](const uint4& q, float (&f)[8]) {
    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
    if constexpr (kVec == 8) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(w4[e] << 16);
        f[2 * e + 1] = __uint_as_float(w4[e] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(w4[e]);
    }
  };
  float mx = -__builtin_inff();    // ordinary maximum
  float mnan = -__builtin_inff();  // NaN-propagating maximum
  uint32_t at = 0xFFFFFFFFu;       // first chunk of this thread that reached mx
  auto take = [&](const uint4& q, uint32_t ch) {
    float f[8];
    unpack(q, f);
    float lm = __builtin_fmaxf(f[0], f[1]), ln = maximum2f(f[0], f[1]);
#pragma unroll
    for (int e = 2; e < kVec; ++e) {
      lm = __builtin_fmaxf(lm, f[e]);
      ln = maximum2f(ln, f[e]);
    }
    mnan = maximum2f(mnan, ln);
    if (lm > mx) {
      mx = lm;
      at = ch;
    }
  };
  for (uint32_t base = 0; base < nv; base += kGreedyInFlight * kThreads) {
    uint4 d[kGreedyInFlight];
#pragma unroll
    for (int u = 0; u < kGreedyInFlight; ++u) {
      const uint32_t ch = base + (uint32_t)u * kThreads + tid;
      const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(ch * 16u), 0, 2);
      d[u] = ch < nv ? make_uint4(v.x, v.y, v.z, v.w) : make_uint4(kNegInf4, kNegInf4, kNegInf4, kNegInf4);
    }
#pragma unroll
    for (int u = 0; u < kGreedyInFlight; ++u) take(d[u], base + (uint32_t)u * kThreads + tid);
  }
  // The ragged end (V not a multiple of the chunk), one element per thread.
  float tail_x = -__builtin_inff();
  const uint32_t tail_id = nv * (uint32_t)kVec + tid;
  if ((int64_t)tail_id < a.V) {
    tail_x = E::to_float((uint32_t)row[tail_id]);
    mnan = maximum2f(mnan, tail_x);
  }

  const float M = block_reduce(__builtin_fmaxf(mx, tail_x),
                               [](float x, float y) { return __builtin_fmaxf(x, y); }, red);
  const uint32_t bad = block_reduce((mnan != mnan || mnan == __builtin_inff()) ? 1u : 0u, MaxOp(), red);
  if (bad != 0u) {
    finish_empty_row(a, b, slot, TSC_ROW_NONFINITE);
    return;
  }
  if (M == -__builtin_inff()) {
    finish_empty_row(a, b, slot, TSC_ROW_NO_SUPPORT);
    return;
  }
  uint32_t id = 0xFFFFFFFFu;
  if (at != 0xFFFFFFFFu && mx == M) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(at * 16u), 0, 2);
    float f[8];
    unpack(make_uint4(v.x, v.y, v.z, v.w), f);
#pragma unroll
    for (int e = kVec - 1; e >= 0; --e)
      if (f[e] == M) id = at * (uint32_t)kVec + (uint32_t)e;
  }
  if (tail_x == M && tail_id < id) id = tail_id;
  const uint32_t token = block_reduce(id, MinOp(), red);
  if (tid == 0) {
    a.tokens[b] = (int32_t)token;
    a.row_status[b] = TSC_ROW_OK;
    if (slot >= 0) {
      a.packed_ids[slot * a.W] = (int32_t)token;
      if (a.logprobs) a.logprobs[slot * a.W] = 0.0f;
      a.lengths[slot] = 1;
      a.selected_logprob[slot] = 0.0f;
    }
  }
}

}  // namespace tsc
