// Replay of a captured support under new logits: the log-softmax of the row restricted to the
// support, at the sampled token (vLLM "Sampling Mask / Distribution Replay" article, section
// "RL training side: computing pi_theta with the mask": the training model's logits are masked
// to the support the sampler returned, so that pi_theta and pi_old share one normalizer).
//
// One workgroup per row. The support is either the row's packed ids (a gather of at most W
// logits) or, for a row whose capture overflowed, its bitmask (a pass over ceil(V / 8) mask
// bytes that loads only the chunks of 8 logits holding set bits). Each thread keeps an online
// maximum and sum of exp((x - max) / T) over its share; one block-wide merge of those states,
// then the token's logprob in float64.
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
  float m[kWaves];
  float s[kWaves];
  uint32_t f[kWaves];
  uint32_t scan[kWaves];  // member chunks per wave (staging)
};

// Staging of a bitmask row's member chunks in LDS for the support-logprob pass (bfloat16 rows of
// at most kStageChunks chunks, with at most kStageSlots member chunks): the pass then reads
// each packed id's logit from LDS instead of gathering it from memory again.
constexpr int kStageChunks = 16384;  // V <= 131072
constexpr int kStageSlots = 7168;    // 112 KB of 16-byte chunks
struct ReplayStage {
  uint16_t slot_of[kStageChunks];  // chunk -> its slot, for member chunks only
  uint4 chunk[kStageSlots];
};

// Online log-sum-exp state of one thread: m the largest finite logit seen, s = sum of
// exp2((x - m) * c) over the finite ones (c = log2(e) / T).
struct OnlineLse {
  float m = -__builtin_inff();
  float s = 0.0f;
  uint32_t flags = 0;  // kBad: a NaN or +inf logit; kSeen: an entry of the support
  __device__ inline void add(float x, float c) {
    flags |= kSeen;
    if (x != x || x == __builtin_inff()) {
      flags |= kBad;
    } else if (x > m) {
      s = s * __builtin_amdgcn_exp2f((m - x) * c) + 1.0f;  // m = -inf: s is 0, 0 * 0 + 1
      m = x;
    } else if (x != -__builtin_inff()) {
      s += __builtin_amdgcn_exp2f((x - m) * c);
    }
  }
  // One chunk of 8 logits with the non-members already set to -inf, cm their maximum: one
  // rescale to the new maximum, then one exponential per position, with no branch. A NaN or
  // +inf member leaves s NaN for good (the caller flags it once, after its pass); -inf adds 0.
  __device__ inline void add_masked(const float (&xm)[8], float cm, float c) {
    const float mn = cm > m ? cm : m;
    s *= mn == m ? 1.0f : __builtin_amdgcn_exp2f((m - mn) * c);  // m = -inf: s is 0 and stays 0
    m = mn;
    const float base = m == -__builtin_inff() ? 0.0f : m;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += __builtin_amdgcn_exp2f((xm[e] - base) * c);
  }
  static constexpr uint32_t kBad = 1, kBadId = 2, kFound = 4, kSeen = 8;
};

// (m, s) of two partial states over one scale: the larger maximum, the sums rescaled to it.
__device__ inline void lse_merge(float& m, float& s, float m2, float s2, float c) {
  const float M = m > m2 ? m : m2;
  float r = 0.0f;
  if (m != -__builtin_inff()) r += s * __builtin_amdgcn_exp2f((m - M) * c);
  if (m2 != -__builtin_inff()) r += s2 * __builtin_amdgcn_exp2f((m2 - M) * c);
  m = M;
  s = r;
}

// One workgroup-wide combination of the threads' states (a single barrier): each wave merges
// its lanes with DPP moves, lane 0 stores the wave's state, and every wave merges the 16 wave
// states in the same fixed order.
__device__ inline void lse_block(OnlineLse& st, float c, ReplayShared& sh) {
  float m = st.m, s = st.s;
  uint32_t f = st.flags;
  auto step = [&](auto mv) {
    const float m2 = mv(m), s2 = mv(s);
    lse_merge(m, s, m2, s2, c);
    f |= mv(f);
  };
  step([](auto v) { return dpp_mov<dpp::kQuadSwap1>(v, v); });
  step([](auto v) { return dpp_mov<dpp::kQuadSwap2>(v, v); });
  step([](auto v) { return dpp_mov<dpp::kRowRor4>(v, v); });
  step([](auto v) { return dpp_mov<dpp::kRowRor8>(v, v); });
  {
    // Every lane of a row of 16 now holds that row's state: merge the four rows.
    float rm[4], rs[4];
    uint32_t rf[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      rm[r] = read_lane(m, 16 * r);
      rs[r] = read_lane(s, 16 * r);
      rf[r] = read_lane(f, 16 * r);
    }
    m = rm[0], s = rs[0], f = rf[0];
#pragma unroll
    for (int r = 1; r < 4; ++r) {
      lse_merge(m, s, rm[r], rs[r], c);
      f |= rf[r];
    }
  }
  const uint32_t w = threadIdx.x / kWaveSize;
  if ((threadIdx.x & (kWaveSize - 1)) == 0) {
    sh.m[w] = m;
    sh.s[w] = s;
    sh.f[w] = f;
  }
  lds_barrier();
  // The 16 wave states: lane l reads wave l % 16's (one LDS read per wave instead of 16
  // broadcast reads), the same four DPP merges combine each row of 16, and lane 0 holds the
  // result, the same in every wave.
  const uint32_t l16 = threadIdx.x & (kWaves - 1);
  m = sh.m[l16], s = sh.s[l16], f = sh.f[l16];
  step([](auto v) { return dpp_mov<dpp::kQuadSwap1>(v, v); });
  step([](auto v) { return dpp_mov<dpp::kQuadSwap2>(v, v); });
  step([](auto v) { return dpp_mov<dpp::kRowRor4>(v, v); });
  step([](auto v) { return dpp_mov<dpp::kRowRor8>(v, v); });
  st.m = read_lane(m, 0), st.s = read_lane(s, 0), st.flags = read_lane(f, 0);
}

template <int DT, bool STAGE>
__global__ void __launch_bounds__(kThreads) replay_kernel(ReplayArgs a) {
  using E = Elem<DT>;
  static_assert(!STAGE || DT == TSC_DTYPE_BF16, "staging holds bfloat16 chunks");
  __shared__ ReplayShared sh;
  [[maybe_unused]] ReplayStage* stg = nullptr;
  if constexpr (STAGE) {
    __shared__ ReplayStage stage_lds;
    stg = &stage_lds;
  }
  const int64_t j = blockIdx.x;
  const uint32_t tid = threadIdx.x;
  const auto* row = reinterpret_cast<const typename E::Bits*>(a.logits) + j * a.ld;
  const int64_t V = a.V;
  constexpr bool kHalf = sizeof(typename E::Bits) == 2;
  constexpr int kS = kHalf ? 16 : 8;  // chunks of 8 ids per group of the bitmask pass
  const uint32_t nfull = (uint32_t)(V / 8);  // chunks wholly inside the row

  // Loads whose addresses do not depend on the row's scalars go out with them, so that their
  // latencies overlap: the thread's first packed id and, when rows may come from bitmasks read
  // in groups of kS mask bytes, the thread's first group.
  const int32_t* ids = a.packed_ids + j * a.W;
  const int32_t id_pre = (int32_t)tid < a.W ? ids[tid] : 0;
  const uint8_t* bits_row = a.bits ? a.bits + j * a.bits_ld : nullptr;
  const bool wide = bits_row != nullptr && a.capture_status != nullptr &&
                    (reinterpret_cast<uintptr_t>(row) & 15u) == 0 &&
                    (reinterpret_cast<uintptr_t>(bits_row) & 15u) == 0 && (a.bits_ld & 15) == 0;
  uint32_t bw_pre[kS / 4] = {};
  if (wide && tid * kS < nfull) {  // tid < the number of groups: inside the mask row
    if constexpr (kS == 16) {
      const uint4 mb = *reinterpret_cast<const uint4*>(bits_row + (size_t)tid * kS);
      bw_pre[0] = mb.x, bw_pre[1] = mb.y, bw_pre[2] = mb.z, bw_pre[3] = mb.w;
    } else {
      const uint2 mb = *reinterpret_cast<const uint2*>(bits_row + (size_t)tid * kS);
      bw_pre[0] = mb.x, bw_pre[1] = mb.y;
    }
  }

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
  const bool ok = __builtin_isfinite(T) && T >= 1.1754943508222875e-38f && tok >= 0 && tok < V &&
                  (from_bits ? a.bits != nullptr : n_ok);
  if (!ok) {
    if (tid == 0) {
      a.row_status[j] = TSC_ROW_INVALID_PARAM;
      a.selected_logprob[j] = __builtin_nanf("");
    }
    return;
  }
  // The token's own logit, loaded now so that its latency overlaps the support's.
  const float xt = tid == 0 ? E::to_float((uint32_t)row[tok]) : 0.0f;
  const float c = 1.4426950408889634f / T;
  OnlineLse acc;
  const uint8_t* brow = from_bits ? bits_row : nullptr;  // null: a packed row
  // Staging: the member chunks of the thread's first group take consecutive slots, from a
  // block-wide exclusive scan of their counts (rows of one group per thread only).
  [[maybe_unused]] bool staged_row = false;
  [[maybe_unused]] uint32_t slot_next = 0;
  if constexpr (STAGE) {
    if (from_bits && wide && nfull <= (uint32_t)kStageChunks) {  // uniform over the block
      uint32_t cnt = 0;
#pragma unroll
      for (int q = 0; q < kS; ++q) {
        const uint32_t byte = (bw_pre[q >> 2] >> (8 * (q & 3))) & 0xFFu;
        cnt += (tid * kS + (uint32_t)q < nfull && byte != 0u) ? 1u : 0u;
      }
      const uint32_t incl = wave_incl_scan(cnt, SumOp(), 0u);
      const uint32_t w = tid / kWaveSize;
      if ((tid & (kWaveSize - 1)) == kWaveSize - 1) sh.scan[w] = incl;
      lds_barrier();
      uint32_t total;
      const uint32_t before = waves_prefix(sh.scan, SumOp(), 0u, total);
      slot_next = before + incl - cnt;
      staged_row = total <= (uint32_t)kStageSlots;
    }
  }
  if (!from_bits) {
    // kU entries per thread at a time: their ids, then their logits, load together.
    constexpr int kU = 4;
    for (int32_t i0 = (int32_t)tid; i0 < n; i0 += kThreads * kU) {
      int32_t idv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int32_t i = i0 + u * kThreads;
        idv[u] = i >= n ? -1 : i == (int32_t)tid ? id_pre : ids[i];
      }
      float xv[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u)
        xv[u] = idv[u] >= 0 && idv[u] < V ? E::to_float((uint32_t)row[idv[u]]) : 0.0f;
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        if (i0 + u * kThreads >= n) continue;
        const int32_t id = idv[u];
        if (id < 0 || id >= V) {
          acc.flags |= OnlineLse::kBadId;
          continue;
        }
        if (id == tok) acc.flags |= OnlineLse::kFound;
        acc.add(xv[u], c);
      }
    }
  } else {
    // Chunks of 8 ids, one mask byte each; non-members become -inf, so that every chunk takes
    // the same branch-free update. With a 16-byte aligned row, the mask bytes of kS chunks are
    // read first, then all the chunks with members at once, one 16-byte vector load per chunk
    // of bfloat16 (two of float32). When the mask row is 16-byte aligned too (as the sampler
    // writes them) a thread takes kS consecutive chunks and reads their mask bytes in one load;
    // otherwise it takes chunk c0 + s * kThreads at step s, so that neighbouring lanes read
    // neighbouring mask bytes. Rows that are not aligned, and a last, partial chunk, take
    // element loads.
    constexpr int kV = kHalf ? 1 : 2;  // kS loads of 16 * kV bytes in flight
    uint32_t seen = 0;
    auto update = [&](uint32_t byte, const uint32_t (&fb)[8]) {  // fb: float32 bit patterns
      float xm[8];
      float cm = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t keep = (uint32_t)((int32_t)(byte << (31 - e)) >> 31);  // ones for a member
        xm[e] = __uint_as_float((fb[e] & keep) | (0xFF800000u & ~keep));
        cm = __builtin_fmaxf(cm, xm[e]);
      }
      acc.add_masked(xm, cm, c);
    };
    auto element_chunk = [&](uint32_t ch, uint32_t byte) {
      uint32_t fb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        fb[e] = (byte >> e) & 1u ? __float_as_uint(E::to_float((uint32_t)row[(size_t)ch * 8 + e])) : 0u;
      update(byte, fb);
      seen |= byte;
    };
    if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0) {
      // One pass for each layout, compiled apart, so that each keeps its own simple addressing.
      auto pass = [&](auto layout) {
      constexpr bool kWide = decltype(layout)::value;
      auto chunk_of = [&](uint32_t g, int s) -> uint32_t {
        return kWide ? g * kS + (uint32_t)s : g + (uint32_t)s * kThreads;
      };
      const uint32_t ngroups = kWide ? (nfull + kS - 1) / kS : nfull;
      const uint32_t gstep = kWide ? kThreads : kThreads * kS;
      for (uint32_t g = tid; g < ngroups; g += gstep) {
        uint32_t bw[kS / 4];  // the kS mask bytes, four to a word
        if constexpr (kWide) {  // bits_ld is a multiple of 16: the whole group lies inside the mask row
          if (g == tid) {
#pragma unroll
            for (int q = 0; q < kS / 4; ++q) bw[q] = bw_pre[q];
          } else if constexpr (kS == 16) {
            const uint4 mb = *reinterpret_cast<const uint4*>(brow + (size_t)g * kS);
            bw[0] = mb.x, bw[1] = mb.y, bw[2] = mb.z, bw[3] = mb.w;
          } else {
            const uint2 mb = *reinterpret_cast<const uint2*>(brow + (size_t)g * kS);
            bw[0] = mb.x, bw[1] = mb.y;
          }
        } else {
#pragma unroll
          for (int q = 0; q < kS / 4; ++q) bw[q] = 0u;
#pragma unroll
          for (int s = 0; s < kS; ++s) {
            const uint32_t ch = chunk_of(g, s);
            bw[s >> 2] |= (ch < nfull ? (uint32_t)brow[ch] : 0u) << (8 * (s & 3));
          }
        }
#pragma unroll
        for (int s = 0; s < kS; ++s)  // chunks past the full ones: none
          if (chunk_of(g, s) >= nfull) bw[s >> 2] &= ~(0xFFu << (8 * (s & 3)));
#pragma unroll
        for (int q = 0; q < kS / 4; ++q) seen |= bw[q];
        auto byte_of = [&](int s) -> uint32_t { return (bw[s >> 2] >> (8 * (s & 3))) & 0xFFu; };
        {
          uint4 raw[kS][kV] = {};  // chunks without members stay 0; their positions are masked
#pragma unroll
          for (int u = 0; u < kS; ++u) {
            if (byte_of(u) != 0u) {
              const uint32_t ch = chunk_of(g, u);
#pragma unroll
              for (int h = 0; h < kV; ++h)
                raw[u][h] = *reinterpret_cast<const uint4*>(row + (size_t)ch * 8 + 4 * h);
            }
          }
          if constexpr (STAGE && kWide) {
            if (staged_row) {  // one group per thread: this is the thread's first
#pragma unroll
              for (int u = 0; u < kS; ++u) {
                if (byte_of(u) != 0u) {
                  const uint32_t ch = chunk_of(g, u);
                  stg->chunk[slot_next] = raw[u][0];
                  stg->slot_of[ch] = (uint16_t)slot_next;
                  ++slot_next;
                }
              }
            }
          }
#pragma unroll
          for (int u = 0; u < kS; ++u) {
            uint32_t fb[8];
            if constexpr (kHalf) {
              const uint32_t w4[4] = {raw[u][0].x, raw[u][0].y, raw[u][0].z, raw[u][0].w};
#pragma unroll
              for (int e = 0; e < 8; ++e) fb[e] = (e & 1) ? (w4[e >> 1] & 0xFFFF0000u) : (w4[e >> 1] << 16);
            } else {
              const uint32_t w8[8] = {raw[u][0].x, raw[u][0].y, raw[u][0].z, raw[u][0].w,
                                      raw[u][kV - 1].x, raw[u][kV - 1].y, raw[u][kV - 1].z,
                                      raw[u][kV - 1].w};
#pragma unroll
              for (int e = 0; e < 8; ++e) fb[e] = w8[e];
            }
            update(byte_of(u), fb);  // a chunk without members adds 0
          }
        }
      }
      };
      if (wide)
        pass(BoolTag<true>{});
      else
        pass(BoolTag<false>{});
    } else {
      for (uint32_t ch = tid; ch < nfull; ch += kThreads) {
        const uint32_t byte = brow[ch];
        if (byte != 0u) element_chunk(ch, byte);
      }
    }
    if ((V & 7) && tid == kThreads - 1) element_chunk(nfull, brow[nfull] & ((1u << (V & 7)) - 1u));
    if (seen != 0u) acc.flags |= OnlineLse::kSeen;
    if (!(acc.s == acc.s) || acc.m == __builtin_inff()) acc.flags |= OnlineLse::kBad;
    if (tid == 0 && ((brow[tok >> 3] >> (tok & 7)) & 1u)) acc.flags |= OnlineLse::kFound;
  }
  lse_block(acc, c, sh);
  const float M = acc.m;
  const uint32_t flags = acc.flags;
  int8_t status = TSC_ROW_OK;
  if ((flags & OnlineLse::kBadId) || !(flags & OnlineLse::kSeen)) status = TSC_ROW_INVALID_PARAM;
  else if (flags & OnlineLse::kBad) status = TSC_ROW_NONFINITE;
  else if (M == -__builtin_inff()) status = TSC_ROW_NO_SUPPORT;
  const double lnS = log((double)acc.s);
  if (tid == 0) {
    a.row_status[j] = status;
    float sel = __builtin_nanf("");
    if (status == TSC_ROW_OK)
      sel = (flags & OnlineLse::kFound) ? (float)(((double)xt - (double)M) / (double)T - lnS)
                                        : -__builtin_inff();
    a.selected_logprob[j] = sel;
  }
  // The logprob of every packed entry (for an overflowing row, of its packed prefix). A thread
  // takes kU entries at a time: their ids load together, then their logits (and mask bytes)
  // together, so that a row of W entries costs a few round trips, not two per entry.
  if (a.logprobs != nullptr && status == TSC_ROW_OK && n_ok) {
    constexpr int kU = 8;
    float* out = a.logprobs + j * a.W;
    // A row of at least kNtStoreMin logprobs is written with nontemporal stores, so that it
    // streams to memory instead of staying dirty in L2 for the kernel's end to write back; the
    // two store kinds are separate instantiations of the loop (a run-time choice between two
    // otherwise equal stores is merged by the compiler into one ordinary store).
    auto lp_pass = [&](auto nt_tag) {
      constexpr bool kNt = decltype(nt_tag)::value;
      for (int32_t i0 = (int32_t)tid; i0 < n; i0 += kThreads * kU) {
        int32_t idv[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int32_t i = i0 + u * kThreads;
          idv[u] = i >= n ? -1 : i == (int32_t)tid ? id_pre : ids[i];
        }
        float xv[kU];
        uint32_t bv[kU];
        if (STAGE && staged_row) {  // members of full chunks: their logits from the LDS stage
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const int32_t id = idv[u];
            bv[u] = id >= 0 && id < V ? (uint32_t)brow[id >> 3] : 0u;
          }
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const int32_t id = idv[u];
            const uint32_t ch = (uint32_t)id >> 3;
            float x = -__builtin_inff();
            if ((bv[u] >> (id & 7)) & 1u) {
              if (ch < nfull) {
                const uint16_t* st16 = reinterpret_cast<const uint16_t*>(stg->chunk);
                x = E::to_float((uint32_t)st16[(uint32_t)stg->slot_of[ch] * 8u + (uint32_t)(id & 7)]);
              } else {
                x = E::to_float((uint32_t)row[id]);  // the ragged last chunk is not staged
              }
            }
            xv[u] = x;
          }
        } else {
#pragma unroll
          for (int u = 0; u < kU; ++u) {
            const int32_t id = idv[u];
            const bool ok = id >= 0 && id < V;
            xv[u] = ok ? E::to_float((uint32_t)row[id]) : -__builtin_inff();
            bv[u] = ok ? (brow == nullptr ? 0xFFu : (uint32_t)brow[id >> 3]) : 0u;
          }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int32_t i = i0 + u * kThreads;
          if (i >= n) continue;
          // Masked log-softmax: an id outside the support (possible only in a bitmask row) is -inf.
          const bool in = (bv[u] >> (idv[u] & 7)) & 1u;
          const float x = in ? xv[u] : -__builtin_inff();
          const float lp = (float)(((double)x - (double)M) / (double)T - lnS);
          if constexpr (kNt)
            __builtin_nontemporal_store(lp, &out[i]);
          else
            out[i] = lp;
        }
      }
    };
    if (n >= (int32_t)kNtStoreMin)
      lp_pass(BoolTag<true>{});
    else
      lp_pass(BoolTag<false>{});
  }
}

}  // namespace tsc
