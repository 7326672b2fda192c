// Single-read sampler path for float32 rows (one 1024-thread workgroup per row).
//
// A float32 key is 32 bits wide, so the per-key histograms of the bfloat16 path do not apply.
// Here the row is still read exactly once, and the candidates are ordered by a sort instead:
//   1. Stream. The lane maxima of every segment's first two loads give the mass reference R and
//      a cutoff theta over the keys' top 16 bits, set safely below the k-th largest value (the
//      sampled maximum of rank mu + 5 sd + 6, below) or, when higher, at the min-p floor
//      R + T ln(min_p) below which no token passes min-p; every 16-byte load (4 values) whose
//      maximum reaches theta is stashed whole in LDS, and (top_p < 1) each lane sums
//      exp2(x log2(e) / T - R log2(e) / T).
//   2. Each wave expands its stash into sort words (key << 32 | ~id) of the values >= theta,
//      appended to one candidate array of the row (order does not matter: it is sorted next).
//   3. A bitonic sort of the candidates in LDS into (value descending, id ascending) order; the
//      stages whose pairs lie within 128 entries stay inside one wave (no workgroup barrier).
//   4. In sorted order: weights exp((x - m) / T) in float64, their exclusive prefix (a block
//      scan), tie groups (equal keys), and the joint predicates at each group's first entry:
//      fewer than k entries before it, prefix mass <= top_p * Z, (x - m) / T >= ln(min_p). The
//      support is the entries before the first failing group. Every token >= theta is a
//      candidate, so this is exact for the candidates; the row is decided here iff at least k
//      candidates exist, a candidate group fails (then every smaller token fails as well), or
//      the value just below theta fails min-p.
//   5. The race in float64 over the support (score (x - m) / T - ln(-ln u), ties to the lowest
//      id), the logprobs (x - m) / T - ln Z_S, and the capture: the sorted prefix itself.
// Rows this path cannot decide exactly (capacities, theta above the support's end, a mass sum
// that overflows) return false and run through general_row in the same workgroup.
#pragma once

namespace tsc {

constexpr int kF32ShortLoads = 8;    // 16-byte loads per lane: rows up to 32768 values
constexpr int kF32LongLoads = 32;    // rows up to 131072 values
constexpr int kF32LoadsAhead = 4;    // loads in flight per lane
constexpr int64_t kF32MinV = 8192;
constexpr int64_t kF32ShortMaxV = (int64_t)kWaves * kWaveSize * kF32ShortLoads * 4;  // 32768
constexpr int64_t kF32MaxV = (int64_t)kWaves * kWaveSize * kF32LongLoads * 4;       // 131072
constexpr int32_t kF32MaxK = 2048;   // the largest top_k served with a margin over its k-th value
// top_k above kF32MaxK (or off) with top-p or min-p: theta is chosen as for this top_k, which
// leaves about as many candidates as the row's top-p or min-p support needs room for.
constexpr int32_t kF32OffK = 1792;
constexpr uint32_t kF32StashPerWave = 256;
constexpr uint32_t kF32CandCap = 4096;  // sorted candidates (u64 sort words); 4 per thread

struct LayoutF32 {
  static constexpr int kOffStash = 0;                                     // uint4 [16][256]
  static constexpr int kOffStashCh = kWaves * kF32StashPerWave * 16;      // u32 [16][256]
  static constexpr int kOffCand = kOffStashCh + kWaves * kF32StashPerWave * 4;  // u64 [4096]
  static constexpr int kEnd = kOffCand + (int)kF32CandCap * 8;
};
// Per-wave partials of the float32 path, after its LDS regions.
struct F32Scalars {
  double wave_d[kWaves];
  float wave_f[kWaves];
  uint32_t wave_u[kWaves];
  uint32_t ncand;
  double scan_w[kWaves];  // per-wave sums of the sorted weights
  double fail_c[kWaves];  // prefix mass before the wave's first failing group
  uint32_t fail_i[kWaves];  // index of the wave's first failing group (ntot: none)
  double race_s[kWaves];  // the wave's best race score
  uint32_t race_i[kWaves];  // the lowest id holding it
  uint32_t decided;       // rows of at most kF32OneWaveMax candidates: decided by wave 0
};
// Rows with at most this many candidates are sorted, scanned and raced by one wave.
constexpr uint32_t kF32OneWaveMax = 256;
static_assert((size_t)LayoutF32::kEnd + sizeof(F32Scalars) <= kFastDynLds,
              "the float32 layout fits the buffer");

// One stage (pairs J apart) of a bitonic merge of size kk over a 128-entry block held in
// registers: entry lane in v0, entry lane + 64 in v1, base = the block's first index. A pair's
// lower entry keeps the larger sort word when bit kk of the lower index is clear (that part of
// the sequence sorts descending), else the smaller one.
template <uint32_t J>
__device__ inline void bitonic_stage(uint64_t& v0, uint64_t& v1, uint32_t base, uint32_t kk) {
  const uint32_t lane = threadIdx.x & (kWaveSize - 1);
  if constexpr (J == 64) {  // pair (lane, lane + 64)
    const bool desc = ((base + lane) & kk) == 0u;
    const uint64_t hi = v0 > v1 ? v0 : v1, lo = v0 > v1 ? v1 : v0;
    v0 = desc ? hi : lo;
    v1 = desc ? lo : hi;
  } else {
    const uint32_t low = lane & ~J;
    const bool lower = (lane & J) == 0u;
    const uint64_t o0 = xor_lanes<(int)J>(v0), o1 = xor_lanes<(int)J>(v1);
    const bool max0 = lower == (((base + low) & kk) == 0u);
    const bool max1 = lower == (((base + 64u + low) & kk) == 0u);
    v0 = max0 == (v0 > o0) ? v0 : o0;
    v1 = max1 == (v1 > o1) ? v1 : o1;
  }
}

// Stages J = jtop, jtop / 2, ..., 1 (jtop <= 64, uniform) of the merge of size kk.
__device__ inline void bitonic_block(uint64_t& v0, uint64_t& v1, uint32_t base, uint32_t kk,
                                     uint32_t jtop) {
  if (jtop >= 64u) bitonic_stage<64>(v0, v1, base, kk);
  if (jtop >= 32u) bitonic_stage<32>(v0, v1, base, kk);
  if (jtop >= 16u) bitonic_stage<16>(v0, v1, base, kk);
  if (jtop >= 8u) bitonic_stage<8>(v0, v1, base, kk);
  if (jtop >= 4u) bitonic_stage<4>(v0, v1, base, kk);
  if (jtop >= 2u) bitonic_stage<2>(v0, v1, base, kk);
  bitonic_stage<1>(v0, v1, base, kk);
}

template <bool NEED_P, int LOADS, bool BITS>
__device__ __forceinline__ bool fast_row_f32(const SampleArgs& a, int64_t b, int64_t& slot,
                                             float T, int32_t k, int32_t kv, float p, float mp,
                                             uint64_t seed, uint64_t pos, unsigned char* lds,
                                             FastShared& fs) {
  using E = Elem<TSC_DTYPE_F32>;
  using LY = LayoutF32;
  const uint32_t tid = threadIdx.x, lane = lane_id(), wid = wave_id();
  const float* row = reinterpret_cast<const float*>(a.logits) + b * a.ld;
  const uint4* rowv = reinterpret_cast<const uint4*>(row);
  const int64_t V = a.V;
  const uint32_t nch = (uint32_t)(V / 4);
  const uint32_t cw = (nch + kWaves - 1) / kWaves;  // chunks per wave segment
  const uint32_t seg0 = wid * cw;
  const uint32_t seg1 = seg0 + cw < nch ? seg0 + cw : nch;
  const uint32_t nseg = seg1 > seg0 ? seg1 - seg0 : 0u;
  const uint32_t id0 = seg0 * 4u;
  F32Scalars& sc = *reinterpret_cast<F32Scalars*>(lds + LY::kEnd);
  static_assert(LOADS >= kF32LoadsAhead, "the first loads are issued together");

  // Rank of theta among the sampled lane maxima (maxima of 4 values, up to 2048 of them), as on
  // the bfloat16 path: with p_k = 1 - (1 - k/V)^4 and n the sampled chunks, theta is the sampled
  // maximum of rank mu + 5 sd + 6 (mu = n p_k, sd^2 = n p_k (1 - p_k)), which lies above the
  // k-th largest value with probability of the order of 1e-7 or below for independent logits.
  constexpr int kSamples = 2 * kThreads;
  uint32_t theta_rank;
  {
    const float n = (float)(nch < (uint32_t)kSamples ? nch : (uint32_t)kSamples);
    const float t = 1.0f - fminf(1.0f, (float)kv / (float)V);
    const float t2 = t * t;
    const float pk = 1.0f - t2 * t2;
    const float mu = n * pk;
    const float rr = ceilf(mu + 5.0f * sqrtf(mu * (1.0f - pk)) + 6.0f);
    theta_rank = (uint32_t)(rr < 1.0f ? 1.0f : (rr > (float)kSamples ? (float)kSamples : rr));
  }

  __builtin_amdgcn_s_setprio(3);
  uint4 r[LOADS];
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4*>(rowv + seg0), (short)0, (int)(nseg * 16u), 0x00020000);
  const int voff = (int)(lane * 16u);
  auto issue = [&](int j) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, j * kWaveSize * 16, 2);
    r[j] = make_uint4(v.x, v.y, v.z, v.w);
  };
  // The opt-in entry first (loads complete in issue order, so waiting for it never waits for
  // row data), then the first loads of the segment.
  const int32_t opt_e = (a.R <= kThreads && (int64_t)tid < a.R) ? a.optin_rows[tid] : INT32_MIN;
#pragma unroll
  for (int j = 0; j < kF32LoadsAhead && j < LOADS; ++j) issue(j);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  if (tid < (uint32_t)kThetaBins / 2) fs.theta_hist[tid] = 0u;
  if (tid == 0) sc.ncand = 0u;
  const uint32_t nfull = uniform_u32(nseg / kWaveSize);
  constexpr uint32_t kNegInf = 0xFF800000u;
  auto mask_tail = [&](int j) {
    if ((uint32_t)j >= nfull) {
      if ((uint32_t)j * kWaveSize + lane >= nseg) r[j] = make_uint4(kNegInf, kNegInf, kNegInf, kNegInf);
    }
  };
  auto load_max = [](const uint4& q) {
    return maximum3f(__uint_as_float(q.x), __uint_as_float(q.y),
                     maximum2f(__uint_as_float(q.z), __uint_as_float(q.w)));
  };
  // Sample: lane maxima of the first two loads; R = their maximum (the reference of the mass).
  mask_tail(0);
  const float lm0 = load_max(r[0]);
  mask_tail(1);
  const float lm1 = load_max(r[1]);
  {
    const float wm = wave_reduce(maximum2f(lm0, lm1), MaximumF32());
    if (lane == 0) sc.wave_f[wid] = wm;
  }
  // The capture slot's validity scan (opt-in entries loaded before the row) shares the two
  // barriers of the theta selection; its last step reads fs.slot_hit after the stream.
  const bool slot_here = a.R <= kThreads;
  SlotScan sscan{};
  if (slot_here) sscan = slot_step1(opt_e, fs);
  lds_barrier();
  if (slot_here) slot_step2(a, b, sscan, fs);
  const float R = waves_reduce(sc.wave_f, MaximumF32());
  const uint32_t kR = __builtin_isfinite(R) ? key_of<E>(__float_as_uint(R)) >> 16 : 0u;
  {
    // Distances of the sampled maxima below R over the keys' top 16 bits (finite ones only).
    auto add = [&](float v) {
      if (!__builtin_isfinite(v)) return;
      const uint32_t d = kR - (key_of<E>(__float_as_uint(v)) >> 16);
      if (d < (uint32_t)kThetaBins) atomicAdd(&fs.theta_hist[d >> 1], 1u << (16u * (d & 1u)));
    };
    add(lm0);
    add(lm1);
  }
  lds_barrier();
  uint32_t theta_k16;
  {
    constexpr int kPer = kThetaBins / kWaveSize;
    uint32_t hc[kPer];
    uint32_t lsum = 0;
#pragma unroll
    for (int q2 = 0; q2 < kPer / 2; ++q2) {
      const uint32_t two = fs.theta_hist[lane * (kPer / 2) + q2];
      hc[2 * q2] = two & 0xFFFFu;
      hc[2 * q2 + 1] = two >> 16;
      lsum += hc[2 * q2] + hc[2 * q2 + 1];
    }
    uint32_t tot;
    uint32_t run = wave_excl_sum(lsum, tot);
    uint32_t found = 0xFFFFFFFFu;
#pragma unroll
    for (int q4 = 0; q4 < kPer; ++q4) {
      run += hc[q4];
      if (found == 0xFFFFFFFFu && run >= theta_rank) found = lane * kPer + q4;
    }
    const uint32_t dmin = wave_reduce(found, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
    const uint32_t dsel = dmin != 0xFFFFFFFFu ? dmin : (uint32_t)kThetaBins - 1u;
    theta_k16 = uniform_u32(kR > dsel ? kR - dsel : 0u);
  }
  // Min-p floor, as on the bfloat16 path: no token below R + T ln(min_p) is in the support (the
  // row maximum is at least R), so theta rises to that floor (2^-16 of its terms lower, more than
  // the rounding of the float computation and of the scans' min-p test) when it is higher. The
  // lowest value of a 16-bit key prefix lies at or below every value with that prefix.
  if (mp > 0.0f) {
    const float lnmp = __logf(mp);
    const float floor_v = R + T * lnmp - (__builtin_fabsf(R) + T * __builtin_fabsf(lnmp) + T) * 0x1p-16f;
    if (__builtin_isfinite(floor_v)) {
      const uint32_t fk16 = key_of<E>(__float_as_uint(floor_v)) >> 16;
      theta_k16 = uniform_u32(fk16 > theta_k16 ? fk16 : theta_k16);
    }
  }
  // Candidates: values whose key's top 16 bits reach theta_k16, i.e. values >= theta.
  const float theta = E::to_float(bits_of_key<E>(theta_k16 << 16));
  // True when the value just below theta fails the scans' min-p test: then every token below
  // theta does, and the candidates hold the whole support whatever k is.
  auto below_theta_fails_min_p = [&](double dm, double dT, double ln_mp) {
    if (!(mp > 0.0f) || theta_k16 == 0u) return false;
    const float xb = E::to_float(bits_of_key<E>((theta_k16 << 16) - 1u));
    return !(((double)xb - dm) / dT >= ln_mp);
  };
  const float th = theta > -3.4028234663852886e38f ? theta : -3.4028234663852886e38f;

  // ---- Stream: running maximum, mass, stash of the loads that may hold a candidate -----------
  const float c = 1.4426950408889634f / T;
  const float nrc = uniform_f32(__builtin_isfinite(R) ? -R * c : 0.0f);
  float m_l = maximum2f(lm0, lm1);
  float s_a = 0.0f, s_b = 0.0f;
  uint4* stash = reinterpret_cast<uint4*>(lds + LY::kOffStash) + wid * kF32StashPerWave;
  uint32_t* stash_ch = reinterpret_cast<uint32_t*>(lds + LY::kOffStashCh) + wid * kF32StashPerWave;
  uint32_t wcnt = 0;  // flagged loads of the wave (wave-uniform); past the stash: fallback
  auto step = [&](int j, float lm) {
    const uint4& q = r[j];
    if constexpr (NEED_P) {
      const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(__uint_as_float(q.x), c, nrc));
      const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(__uint_as_float(q.y), c, nrc));
      const float e2 = __builtin_amdgcn_exp2f(__builtin_fmaf(__uint_as_float(q.z), c, nrc));
      const float e3 = __builtin_amdgcn_exp2f(__builtin_fmaf(__uint_as_float(q.w), c, nrc));
      if (j & 1) s_b += (e0 + e1) + (e2 + e3);
      else s_a += (e0 + e1) + (e2 + e3);
    }
    const bool flag = lm >= th;  // NaN fails
    const uint64_t mask = __ballot(flag);
    const uint32_t n = (uint32_t)__popcll(mask);
    if (n != 0u) {
      if (wcnt + n <= kF32StashPerWave && flag) {
        const uint32_t at = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)mask, wcnt));
        stash[at] = q;
        stash_ch[at] = (uint32_t)j * kWaveSize + lane;
      }
      wcnt += n;
    }
    asm volatile("" : "+v"(s_a), "+v"(s_b), "+v"(m_l));
  };
  step(0, lm0);
  step(1, lm1);
  // Loads 0-3 went out together; step 2 issues loads 4 and 5, every later step j load j + 3, so
  // that four loads are in flight while one is used.
#pragma unroll
  for (int j = 2; j < LOADS; ++j) {
    if (j == 2 && kF32LoadsAhead < LOADS) issue(kF32LoadsAhead);
    if (j + 3 < LOADS && j + 3 > kF32LoadsAhead) issue(j + 3);
    mask_tail(j);
    const float lm = load_max(r[j]);
    m_l = maximum2f(m_l, lm);
    step(j, lm);
  }

  // ---- Per wave: partials, then its stash expanded into the row's candidate array ---------------
  __builtin_amdgcn_s_setprio(2);
  const bool stash_over = wcnt > kF32StashPerWave;
  {
    const float wm = wave_reduce(m_l, MaximumF32());
    double wz = 0.0;
    if constexpr (NEED_P) wz = wave_reduce((double)(s_a + s_b), SumF64());
    if (lane == 0) {
      sc.wave_f[wid] = wm;
      // A reference past kMassRefMax: an infinite mass sends the row to the general path.
      sc.wave_d[wid] = !NEED_P || __builtin_fabsf(nrc) <= kMassRefMax ? wz : __builtin_inf();
      sc.wave_u[wid] = stash_over ? 1u : 0u;
    }
  }
  uint64_t* cand = reinterpret_cast<uint64_t*>(lds + LY::kOffCand);
  if (!stash_over) {
    for (uint32_t base = 0; base < wcnt; base += kWaveSize) {
      const uint32_t i = base + lane;
      uint4 q = make_uint4(kNegInf, kNegInf, kNegInf, kNegInf);
      uint32_t ch = 0;
      if (i < wcnt) {
        q = stash[i];
        ch = stash_ch[i];
      }
      const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
      uint32_t n = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) n += __uint_as_float(w4[e]) >= th ? 1u : 0u;
      uint32_t total;
      const uint32_t off = wave_excl_sum(n, total);
      uint32_t at0 = 0;
      if (lane == 0 && total != 0u) at0 = atomicAdd(&sc.ncand, total);
      uint32_t at = read_lane(at0, 0) + off;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (__uint_as_float(w4[e]) >= th) {
          if (at < kF32CandCap) {
            const uint32_t id = id0 + ch * 4u + (uint32_t)e;
            cand[at] = ((uint64_t)key_of<E>(w4[e]) << 32) | (uint64_t)(~id);
          }
          ++at;
        }
      }
    }
  }
  lds_barrier();  // candidates, partials and the slot scan's per-wave hits are complete
  if (slot_here) {
    slot = slot_step3(fs);
  } else {
    slot = find_capture_slot(a, b, fs.red);
    lds_barrier();
  }

  // ---- Row scalars and decisions (every thread alike) ----------------------------------------
  const float m = waves_reduce(sc.wave_f, MaximumF32());
  const double zr = waves_reduce(sc.wave_d, SumF64());
  const uint32_t over_any = waves_reduce(sc.wave_u, OrU32());
  const uint32_t ntot = uniform_u32(sc.ncand);
  if (!(m == m) || m == __builtin_inff() || !(zr == zr)) {
    finish_empty_row(a, b, slot, TSC_ROW_NONFINITE);
    return true;
  }
  if (m == -__builtin_inff()) {
    finish_empty_row(a, b, slot, TSC_ROW_NO_SUPPORT);
    return true;
  }
  if (over_any != 0u || ntot > kF32CandCap || ntot == 0u || !(zr <= 1.0e300)) return false;
  // Z relative to the maximum: exp2(x c - m c) = exp2(x c - R c) * exp2(R c - m c), with the
  // rounded R c of the stream, so that its rounding cancels.
  const double Z = NEED_P ? zr * exp2_fast(-(double)nrc - (double)m * (double)c) : 0.0;

  // ---- Rows of at most kF32OneWaveMax candidates: one wave decides the row -------------------
  // With so few candidates the workgroup-wide phases below are mostly barrier latency. Wave 0
  // holds the candidates in registers, four per lane (entry lane + 64 r), sorts them, scans
  // their weights, decides the support and races it, and writes every output; the other waves
  // wait at one barrier for its decision (a row it cannot decide goes to the general path, which
  // needs every wave). The arithmetic is that of the workgroup-wide phases, entry for entry.
  if (ntot <= kF32OneWaveMax) {
    auto one_wave = [&]() -> uint32_t {
      uint64_t v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t i = lane + (uint32_t)r * kWaveSize;
        v[r] = i < ntot ? cand[i] : 0ull;  // 0 sorts below every candidate
      }
      // Bitonic sort, descending: blocks (v0, v1) = entries 0..127 and (v2, v3) = 128..255.
      const bool two = ntot > 128u;
#pragma unroll
      for (uint32_t kk = 2u; kk <= 128u; kk <<= 1) {
        bitonic_block(v[0], v[1], 0u, kk, kk >> 1);
        if (two) bitonic_block(v[2], v[3], 128u, kk, kk >> 1);
      }
      if (two) {  // the merge of size 256: entry i against i + 128, then within the blocks
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          const uint64_t hi = v[r] > v[r + 2] ? v[r] : v[r + 2], lo = v[r] > v[r + 2] ? v[r + 2] : v[r];
          v[r] = hi;
          v[r + 2] = lo;
        }
        bitonic_block(v[0], v[1], 0u, 256u, 64u);
        bitonic_block(v[2], v[3], 128u, 256u, 64u);
      }
      // Weights, their exclusive prefix in sorted order, and the first failing tie group.
      const double dm = (double)m, dT = (double)T;
      const double pz = (double)p * Z;
      const bool need_m = mp > 0.0f;
      const double ln_mp = need_m ? log((double)mp) : 0.0;
      const double l2e_T = 1.4426950408889634 / dT;
      double carry = 0.0, zs = 0.0;
      uint32_t L = ntot, prev_last = 0u;
      bool found = false;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t i = lane + (uint32_t)r * kWaveSize;
        const bool in = i < ntot;
        const uint32_t key = (uint32_t)(v[r] >> 32);
        const float x = E::to_float(bits_of_key<E>(key));
        const double w = in ? exp2_fast(((double)x - dm) * l2e_T) : 0.0;  // exp((x - m) / T)
        const double winc = wave_incl_scan(w, [](double p0, double p1) { return p0 + p1; }, 0.0);
        const double C = carry + (winc - w);
        const uint32_t up = __shfl_up(key, 1u, kWaveSize);
        const uint32_t pkey = lane == 0u ? prev_last : up;
        const bool start = in && (i == 0u || key != pkey);
        bool qual = (int64_t)i < (int64_t)k;
        if (NEED_P) qual = qual && C <= pz;
        if (need_m) qual = qual && ((double)x - dm) / dT >= ln_mp;
        const uint64_t fails = __ballot(start && !qual);
        if (!found && fails != 0ull) {
          const int src = (int)__builtin_ctzll(fails);
          L = (uint32_t)r * kWaveSize + (uint32_t)src;
          zs = read_lane(C, src);
          found = true;
        }
        carry += read_lane(winc, kWaveSize - 1);
        prev_last = read_lane(key, kWaveSize - 1);
      }
      if (!found) zs = carry;
      // Decided here iff theta lies at or below the k-th largest value, a candidate group fails,
      // or every token below theta fails min-p.
      if (!(L < ntot || ntot >= (uint32_t)k || below_theta_fails_min_p(dm, dT, ln_mp))) return 0u;
      const double lnzs = log(zs);
      // The race over the support, as in the workgroup-wide phase: float32 scores, the entries
      // within kRaceMargin of the best rescored in float64, ties to the lowest id.
      const float invT = 1.0f / T;
      float best32 = -__builtin_inff();
      uint32_t uw[4];
      float xv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t i = lane + (uint32_t)r * kWaveSize;
        uw[r] = 0u;
        xv[r] = -__builtin_inff();
        if (i < L) {
          uw[r] = race_word(~(uint32_t)v[r], seed, pos);
          xv[r] = E::to_float(bits_of_key<E>((uint32_t)(v[r] >> 32)));
          const float s32 = (xv[r] - m) * invT + race_noise((float)(2u * (uw[r] >> 9) + 1u) * 0x1p-24f);
          best32 = s32 > best32 ? s32 : best32;
        }
      }
      const float top32 = wave_reduce(best32, MaxOp());
      double best = -__builtin_inf();
      uint32_t best_id = 0xFFFFFFFFu;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t i = lane + (uint32_t)r * kWaveSize;
        if (i < L) {
          const uint32_t id = ~(uint32_t)v[r];
          const double u = (double)(2u * (uw[r] >> 9) + 1u) * 0x1p-24;
          if ((xv[r] - m) * invT + race_noise((float)u) >= top32 - kRaceMargin) {
            const double sc_ = ((double)xv[r] - dm) / dT - log(-log(u));
            if (sc_ > best || (sc_ == best && id < best_id)) {
              best = sc_;
              best_id = id;
            }
          }
        }
      }
      const double wbest = wave_reduce(best, MaxOp());
      const uint32_t token = wave_reduce(best == wbest ? best_id : 0xFFFFFFFFu, MinOp());
      // Outputs: the capture, its bitmask when wider than W, then the token's entry.
      const bool capture = slot >= 0;
      const uint32_t W = (uint32_t)a.W;
      if (capture) {
        int32_t* out_ids = a.packed_ids + slot * a.W;
        float* out_lp = a.logprobs ? a.logprobs + slot * a.W : nullptr;
        const uint32_t n = L < W ? L : W;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t i = lane + (uint32_t)r * kWaveSize;
          if (i < n) {
            out_ids[i] = (int32_t)(~(uint32_t)v[r]);
            if (out_lp) out_lp[i] = logprob_of(E::to_float(bits_of_key<E>((uint32_t)(v[r] >> 32))), m, T, lnzs);
          }
        }
        if (BITS && L > W && a.bits != nullptr) {
          // The row cleared, its stores drained, then one atomic OR per support token.
          uint32_t* brow = a.bits + slot * a.bits_ld;
          const uint32_t nw = (uint32_t)bitmask_words(V);
          for (uint32_t i = lane; i < nw; i += kWaveSize) brow[i] = 0u;
          __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const uint32_t i = lane + (uint32_t)r * kWaveSize;
            if (i < L) {
              const uint32_t id = ~(uint32_t)v[r];
              atomicOr(brow + (id >> 5), 1u << (id & 31u));
            }
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t i = lane + (uint32_t)r * kWaveSize;
        if (i < L && ~(uint32_t)v[r] == token) {
          a.tokens[b] = (int32_t)token;
          a.row_status[b] = (capture && L > W) ? TSC_ROW_OVERFLOW : TSC_ROW_OK;
          if (capture) {
            a.lengths[slot] = (int32_t)(L < W ? L : W);
            a.selected_logprob[slot] = logprob_of(xv[r], m, T, lnzs);
          }
        }
      }
      return 1u;
    };
    if (wid == 0) {
      const uint32_t dec = one_wave();
      if (lane == 0) sc.decided = dec;
    }
    lds_barrier();
    return sc.decided != 0u;
  }

  // ---- Sort (descending sort words: value descending, then id ascending) ----------------------
  // Bitonic. Stages whose pairs lie within a 128-entry block run in registers, one block per
  // wave at a time (DPP moves and permlane swaps for pairs less than 64 apart); stages with pairs
  // 128 or more apart run in LDS between workgroup barriers.
  const uint32_t N = uniform_u32(ntot <= 128u ? 128u : 1u << (32 - __builtin_clz(ntot - 1u)));
  for (uint32_t i = ntot + tid; i < N; i += kThreads) cand[i] = 0ull;  // below every candidate
  const uint32_t nblk = N / 128u;
  auto block_pass = [&](uint32_t kk_first, uint32_t kk_last, uint32_t jtop_last) {
    // Merges kk_first..kk_last (each from its own j = kk/2, except the last from jtop_last).
    lds_barrier();
    for (uint32_t blk = wid; blk < nblk; blk += kWaves) {
      const uint32_t base = blk * 128u;
      uint64_t v0 = cand[base + lane], v1 = cand[base + 64u + lane];
      for (uint32_t kk = kk_first; kk <= kk_last; kk <<= 1)
        bitonic_block(v0, v1, base, kk, kk == kk_last ? jtop_last : (kk >> 1));
      cand[base + lane] = v0;
      cand[base + 64u + lane] = v1;
    }
  };
  block_pass(2u, 128u, 64u);
  for (uint32_t kk = 256u; kk <= N; kk <<= 1) {
    for (uint32_t j = kk >> 1; j >= 128u; j >>= 1) {
      lds_barrier();
      const uint32_t lj = 31u - (uint32_t)__builtin_clz(j);
      for (uint32_t t = tid; t < N / 2; t += kThreads) {
        const uint32_t lo = ((t >> lj) << (lj + 1u)) | (t & (j - 1u)), hi = lo + j;
        const uint64_t x = cand[lo], y = cand[hi];
        const bool desc = (lo & kk) == 0u;
        if (desc ? x < y : x > y) {
          cand[lo] = y;
          cand[hi] = x;
        }
      }
    }
    block_pass(kk, kk, 64u);
  }
  lds_barrier();

  // ---- Weights, prefix mass, tie groups and the joint predicates (4 entries per thread) --------
  const double dm = (double)m, dT = (double)T;
  const double pz = (double)p * Z;
  const bool need_m = mp > 0.0f;
  const double ln_mp = need_m ? log((double)mp) : 0.0;
  uint64_t wk[4];
  double wv[4];
  double lsum = 0.0;
  const double l2e_T = 1.4426950408889634 / dT;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t i = tid * 4u + (uint32_t)e;
    wk[e] = 0ull;
    wv[e] = 0.0;
    if (i < ntot) {
      wk[e] = cand[i];
      const float x = E::to_float(bits_of_key<E>((uint32_t)(wk[e] >> 32)));
      wv[e] = exp2_fast(((double)x - dm) * l2e_T);  // exp((x - m) / T), relative error ~2e-7
    }
    lsum += wv[e];
  }
  const uint64_t prev = tid * 4u >= 1u && tid * 4u - 1u < ntot ? cand[tid * 4u - 1u] : 0ull;
  // Exclusive prefix of the weights in sorted order: a wave scan, then the waves before.
  const double winc = wave_incl_scan(lsum, [](double x, double y) { return x + y; }, 0.0);
  if (lane == kWaveSize - 1) sc.scan_w[wid] = winc;
  lds_barrier();
  double total;
  double C = waves_prefix(sc.scan_w, SumF64(), 0.0, total) + (winc - lsum);
  uint32_t first_fail = ntot;
  double c_fail = 0.0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t i = tid * 4u + (uint32_t)e;
    if (i < ntot) {
      const uint32_t key = (uint32_t)(wk[e] >> 32);
      const uint32_t pkey = e == 0 ? (uint32_t)(prev >> 32) : (uint32_t)(wk[e - 1] >> 32);
      const bool start = i == 0u || key != pkey;
      if (start) {
        const float x = E::to_float(bits_of_key<E>(key));
        bool qual = (int64_t)i < (int64_t)k;
        if (NEED_P) qual = qual && C <= pz;
        if (need_m) qual = qual && ((double)x - dm) / dT >= ln_mp;
        if (!qual && first_fail == ntot) {
          first_fail = i;
          c_fail = C;
        }
      }
    }
    C += wv[e];
  }
  // The first failing group of the row lies in the first wave that has one, at its lowest lane
  // with one (indices grow with the thread); the weights before it sum to Z_S.
  {
    const uint64_t fails = __ballot(first_fail < ntot);
    const int src = fails != 0ull ? (int)__builtin_ctzll(fails) : 0;
    const uint32_t wi = fails != 0ull ? read_lane(first_fail, src) : ntot;
    const double wc = read_lane(c_fail, src);
    if (lane == 0) {
      sc.fail_i[wid] = wi;
      sc.fail_c[wid] = wc;
    }
  }
  lds_barrier();
  uint32_t L = ntot;
  double zs = total;
  {
    const uint32_t fi = sc.fail_i[lane & (kWaves - 1)];
    const double fc = sc.fail_c[lane & (kWaves - 1)];
    const uint64_t fails = __ballot(fi < ntot) & 0xFFFFull;  // one lane per wave
    if (fails != 0ull) {
      const int src = (int)__builtin_ctzll(fails);
      L = read_lane(fi, src);
      zs = read_lane(fc, src);
    }
  }
  // Decided here iff theta lies at or below the k-th largest value, a candidate group fails, or
  // every token below theta fails min-p.
  if (!(L < ntot || ntot >= (uint32_t)k || below_theta_fails_min_p(dm, dT, ln_mp))) return false;
  const double lnzs = log(zs);

  // ---- Race over the support, in float64: score (x - m) / T - ln(-ln u), ties -> lowest id ----
  // Float32 scores first (within ~3e-6 of exact for every competitive entry, see race_noise);
  // the entries within kRaceMargin of their wave's best are rescored in float64.
  const float invT = 1.0f / T;
  float best32 = -__builtin_inff();
  uint32_t uw[4];  // race words of this thread's support entries (i = tid + 1024 r)
  float xv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t i = tid + (uint32_t)e * kThreads;
    uw[e] = 0u;
    xv[e] = -__builtin_inff();
    if (i < L) {
      const uint64_t w = cand[i];
      uw[e] = race_word(~(uint32_t)w, seed, pos);
      xv[e] = E::to_float(bits_of_key<E>((uint32_t)(w >> 32)));
      const float s32 = (xv[e] - m) * invT + race_noise((float)(2u * (uw[e] >> 9) + 1u) * 0x1p-24f);
      best32 = s32 > best32 ? s32 : best32;
    }
  }
  const float top32 = wave_reduce(best32, MaxOp());
  double best = -__builtin_inf();
  uint32_t best_id = 0xFFFFFFFFu;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t i = tid + (uint32_t)e * kThreads;
    if (i < L) {
      const uint32_t id = ~(uint32_t)cand[i];
      const double u = (double)(2u * (uw[e] >> 9) + 1u) * 0x1p-24;
      if ((xv[e] - m) * invT + race_noise((float)u) >= top32 - kRaceMargin) {
        const double sc_ = ((double)xv[e] - dm) / dT - log(-log(u));
        if (sc_ > best || (sc_ == best && id < best_id)) {
          best = sc_;
          best_id = id;
        }
      }
    }
  }
  {
    const double wbest = wave_reduce(best, MaxOp());
    const uint32_t wid_best = wave_reduce(best == wbest ? best_id : 0xFFFFFFFFu, MinOp());
    if (lane == 0) {
      sc.race_s[wid] = wbest;
      sc.race_i[wid] = wid_best;
    }
  }

  // ---- Outputs ---------------------------------------------------------------------------------
  // The captured support (it does not depend on the token) goes out before the race's exchange.
  const bool capture = slot >= 0;
  const uint32_t W = (uint32_t)a.W;
  if (capture) {
    int32_t* out_ids = a.packed_ids + slot * a.W;
    float* out_lp = a.logprobs ? a.logprobs + slot * a.W : nullptr;
    const uint32_t n = L < W ? L : W;
    for (uint32_t i = tid; i < n; i += kThreads) {
      const uint64_t w = cand[i];
      out_ids[i] = (int32_t)(~(uint32_t)w);
      if (out_lp) out_lp[i] = logprob_of(E::to_float(bits_of_key<E>((uint32_t)(w >> 32))), m, T, lnzs);
    }
    if (BITS && L > W && a.bits != nullptr) {
      // The support as a bitmask: the row cleared, then one atomic OR per support token.
      uint32_t* brow = a.bits + slot * a.bits_ld;
      const uint32_t nw = (uint32_t)bitmask_words(V);
      for (uint32_t i = tid; i < nw; i += kThreads) brow[i] = 0u;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      for (uint32_t i = tid; i < L; i += kThreads) {
        const uint32_t id = ~(uint32_t)cand[i];
        atomicOr(brow + (id >> 5), 1u << (id & 31u));
      }
    }
  }
  lds_barrier();
  uint32_t token;
  {
    const double s_w = sc.race_s[lane & (kWaves - 1)];
    const uint32_t i_w = sc.race_i[lane & (kWaves - 1)];
    const double top = row16_reduce(s_w, MaxOp());
    token = row16_reduce(s_w == top ? i_w : 0xFFFFFFFFu, MinOp());
  }
  // The token's entry: its logprob, from the same function as the packed entries.
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t i = tid + (uint32_t)e * kThreads;
    if (i < L && ~(uint32_t)cand[i] == token) {
      a.tokens[b] = (int32_t)token;
      a.row_status[b] = (capture && L > W) ? TSC_ROW_OVERFLOW : TSC_ROW_OK;
      if (capture) {
        a.lengths[slot] = (int32_t)(L < W ? L : W);
        a.selected_logprob[slot] = logprob_of(xv[e], m, T, lnzs);
      }
    }
  }
  return true;
}

}  // namespace tsc
