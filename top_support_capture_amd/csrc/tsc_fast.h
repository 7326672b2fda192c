// Single-read sampler kernel for bfloat16 rows (one 1024-thread workgroup per row).
//
// HBM is the bound: a row is read exactly once through a shallow pipeline of 16-byte loads, and
// all per-element work happens while the loads land. Wave w owns a contiguous segment of the row
// (coalesced 1 KB per load instruction), so everything a wave stashes is in id order.
//
//   1. Stream. The lane maxima of the first loads of every segment (a sample spread over the
//      whole row) give a reference R for the mass and a cutoff theta set safely below the k-th
//      largest value: an LDS histogram of their key distances to the sample's maximum, built
//      over the first stream steps so that the loads keep flowing. With min_p > 0 theta rises
//      to the min-p floor of the sample's maximum when that is higher: no token below it passes
//      min-p.
//   2. As each load lands: running maximum (NaN-propagating, so it also detects NaN), for
//      top_p < 1 the lane sum of exp2(x * log2(e) / T - R * log2(e) / T), and a ballot on "this
//      load's maximum >= theta" that stashes the whole 16-byte load in the wave's LDS stash
//      (or, in compaction mode, appends its values >= theta to the wave's candidate list).
//   3. Each wave, as soon as its segment is done: expands its stash into candidate words
//      (bf16 bits << 16 | offset in the segment), still in id order, counts them into a
//      histogram over key - key(theta) and ranks each among its wave's earlier candidates of
//      the same key.
//   4. After one barrier, no more: wave 0 checks the row and scans the histogram bins from the
//      maximum down: the joint threshold is the largest distance d from the maximum with fewer
//      than k tokens strictly above and (top_p < 1) mass strictly above <= top_p * Z; min-p
//      drops whole bins. The support is decided iff at least k candidates were found, a
//      candidate bin below the support's last one fails a predicate, or the value just below
//      theta fails min-p (checked here). Meanwhile the other waves draw every candidate's race
//      uniform (Philox4x32-10, in jobs claimed from an LDS counter) and keep per bin the largest
//      one (all candidates of a bin share their logit, so that one is the bin's best race score).
//   5. Every wave writes the ordered capture of its own candidates: the bin scan gives each tie
//      group's base position, the ranks and a prefix over the waves the rest. Once every draw
//      is done, wave 0 picks the token over the support's bins (float32 scores, float64 for the
//      few within 1e-4 of the best). Waves wait on LDS flags, not barriers.
// Any row this path cannot serve exactly (capacities, theta above the k-th value, overflow of
// the mass, greedy rows, other dtypes or layouts) runs through general_row in the same workgroup.
#pragma once

#include "tsc_general.h"

namespace tsc {

// 16-byte loads per lane: a segment of at most 20 * 512 values for rows up to 163840, 32 * 512
// for rows up to 262144 (two instantiations, so that shorter rows keep the shorter stream code).
constexpr int kShortLoads = 20;
constexpr int kFastLoads = 32;
constexpr int kLoadsFirst = 2;        // loads issued before the first one is awaited
constexpr int kLoadsAhead = 4;        // software pipeline depth afterwards (loads in flight per lane)
constexpr int kStashPerWave = 256;    // stashed loads per wave (stash mode)
constexpr int kSpillPerWave = 512;    // stash mode: flagged loads past the stash, read again later
constexpr int kDBins = 1024;          // histogram bins over the key span above the cutoff
// Key distances of the sampled maxima below their maximum: heavy-tailed rows (a Zipf-like head
// over a wide vocabulary) need theta over 256 keys (two binades of bf16) below it.
constexpr int kThetaBins = 512;
constexpr int64_t kFastMinV = 16384;
constexpr int64_t kFastMaxV = (int64_t)kWaves * kWaveSize * kFastLoads * 8;     // 262144
constexpr int64_t kShortMaxV = (int64_t)kWaves * kWaveSize * kShortLoads * 8;   // 163840
constexpr int32_t kFastMaxK = 4096;   // stash mode; compaction mode above it
// top_k off (or above the compaction range) with top-p or min-p: theta is chosen as for this
// top_k (about 2800 candidates at V = 262144, 2300 at V = 151936). Such a row needs no margin
// over a k-th value, only room for its top-p or min-p support; a wider cutoff (about 5300
// candidates) overflowed the stash (~330 loads per wave against 256), whose excess is read
// again after the stream. Supports wider than theta's reach leave the row to the general path.
constexpr int32_t kOffK = 1792;
constexpr int32_t kCompactMaxK = 8192;
constexpr float kRaceMargin = 1e-4f;  // float32 race scores are within ~3e-6 of exact
// Waves whose stream ends among the first kOwnDraws draw the race uniforms of their own
// candidates before the exchange (while the last streams and their post-stream work finish).
constexpr uint32_t kOwnDraws = 4;

// Two modes share everything but the way candidates are gathered during the stream:
//   stash mode (top_k <= 4096): a load that may hold a value >= theta is stashed whole in LDS
//     (one ballot per load) and expanded into candidates once the wave's stream has ended; past
//     the stash's capacity a flagged load keeps only its chunk index and is read again then;
//   compaction mode (4096 < top_k <= 8192, where most loads hold candidates): the values >= theta
//     of each load are appended to the wave's candidate list as the load lands.
// Each wave counts its candidates per bin bi = key - theta_key in a table of its own (u16; later
// the exclusive prefix over the earlier waves) and ranks each among its earlier candidates of the
// same bin, before the exchange (stash mode keeps the ranks in LDS, compaction mode in
// registers). Stash mode (small supports) writes the capture directly. Compaction mode (supports
// of thousands) writes each survivor's packed word (id | bi << 18) at its position in an LDS stage
// that is copied out with coalesced stores (positions past the stage are written directly).
constexpr int kTableBytes = kDBins * 2;
constexpr int kMaskBins = 256;        // stash mode: bins with a 64-bit lane mask in the table

// LDS regions after the mode-specific ones (bytes from the dynamic buffer base).
template <int kOffTail>
struct TailLayout {
  static constexpr int kOffBinBest = kOffTail;                            // u64 [1024] race per bin
  static constexpr int kOffDummy = kOffBinBest + kDBins * 8;              // u32 [64] scatter sink
  static constexpr int kOffCnt = kOffDummy + kWaveSize * 4;               // u32 [1024] by key - theta
  static constexpr int kOffBinBase = kOffCnt + kDBins * 4;                // u32 [1024] capture base
  static constexpr int kOffBinS = kOffBinBase + kDBins * 4;               // f64 [1024] (x - m) / T
  static constexpr int kEnd = kOffBinS + kDBins * 8;
};
// Stash mode: the stash, its chunk indices, the candidates. Once a wave has expanded its stash,
// its stash slice holds its table (counts, then lane masks) and its chunk-index slice its
// candidates' ranks.
constexpr int kStashBytes = kWaves * kStashPerWave * 16;
constexpr int kStashChBytes = kWaves * kStashPerWave * 4;
struct LayoutStash
    : TailLayout<kStashBytes + kStashChBytes + kWaves * 512 * 4 + kWaves * kSpillPerWave * 2> {
  static constexpr int kCandCap = 512;                      // candidate words per wave
  static constexpr int kOffStash = 0;                       // uint4 [16][256]
  static constexpr int kOffStashCh = kStashBytes;           // u32 [16][256]
  static constexpr int kOffCand = kOffStashCh + kStashChBytes;  // u32 [16][512]
  static constexpr int kOffSpill = kOffCand + kWaves * kCandCap * 4;  // u16 [16][512] chunks
  static constexpr int kOffTables = kOffStash;              // u16 [1024] + u64 [256] per wave
  static constexpr int kTableStride = kStashPerWave * 16;
  static constexpr int kOffRank = kOffStashCh;              // u16 [16][512]
};
static_assert(kThetaBins % (2 * kWaveSize) == 0 && kThetaBins / 2 <= kThreads, "theta histogram");
static_assert(kTableBytes + kMaskBins * 8 <= LayoutStash::kTableStride, "tables fit a slice");
static_assert(LayoutStash::kCandCap * 2 <= kStashPerWave * 4, "ranks fit a chunk-index slice");
// Compaction mode: the candidates, the tables, the stage.
constexpr int kCompactCap = 1024;
struct LayoutCompact
    : TailLayout<kWaves * kCompactCap * 4 + kWaves * kTableBytes + 8192 * 4> {
  static constexpr int kCandCap = kCompactCap;              // candidate words per wave
  static constexpr int kOffCand = 0;                        // u32 [16][1024]
  static constexpr int kOffTables = kOffCand + kWaves * kCandCap * 4;        // u16 [16][1024]
  static constexpr int kTableStride = kTableBytes;
  static constexpr int kOffStage = kOffTables + kWaves * kTableBytes;        // u32 [8192]
  static constexpr int kStageCap = 8192;
};

constexpr size_t kMaxSz(size_t x, size_t y) { return x > y ? x : y; }
constexpr size_t kFastDynLds = kMaxSz(kMaxSz((size_t)kGeneralDynLds + sizeof(GeneralShared),
                                             (size_t)LayoutStash::kEnd),
                                      (size_t)LayoutCompact::kEnd);

// Outcome of the status checks and the bin scan, published by wave 0.
enum FastDecision : int32_t { kProceed = 0, kNonfinite = 1, kNoSupport = 2, kFallback = 3 };

// Per-wave partial results exchanged through LDS (one barrier per exchange).
struct FastShared {
  uint64_t red[kWaves];
  uint32_t theta_hist[kThetaBins / 2];  // two u16 counts per word: distance 2j low, 2j+1 high
  uint32_t kmax0_w[kWaves];
  uint32_t ndone;              // waves whose stream has ended
  uint32_t scan_ready;          // set by wave 0 once the decision and the bin scan are published
  // Counters in steps of 64 (one per wave):
  uint32_t prefix_done;         // waves that finished their share of the capture offsets
  uint32_t job_next;            // next race-draw job to claim
  uint32_t ready;               // race-draw jobs completed
  uint32_t cap_next;            // next wave's candidate list to capture
  uint32_t staged;              // candidate lists captured into the stage
  uint32_t copy_next;           // next slice of the stage to copy out
  uint32_t bits_next;           // next wave's candidate list to set bitmask bits from
  uint32_t bin_hi[kWaves];      // one past the largest bin of the wave's candidates
  uint32_t noise_done[kWaves];  // candidates whose race draws the wave made itself (from the first)
  int32_t slot_wmax[kWaves];
  int32_t slot_hit[kWaves];
  float wave_m[kWaves];
  double wave_z[kWaves];
  uint32_t wave_stash[kWaves];
  uint32_t wave_cand[kWaves];
  int32_t decision;
  int32_t dstar;
  int32_t dlow;                // the largest d (lowest key) holding a candidate
  uint32_t L;
  double lnzs;
  uint32_t aborted;            // set by a wait that reached its limit (see lds_wait_at_least)
};

__device__ inline uint32_t lane_id() { return threadIdx.x & (kWaveSize - 1); }

// Wave index, known to the compiler as wave-uniform (held in a scalar register).
__device__ inline uint32_t wave_id() {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWaveSize));
}

// A value every lane holds alike, moved to a scalar register.
__device__ inline float uniform_f32(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}
__device__ inline uint32_t uniform_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ inline uint32_t mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// The lanes where `in` holds whose bin equals this lane's (bins below 2^nbits, nbits <= 10,
// wave-uniform): one ballot per bit of the bin, and per 32-bit half of the lane mask one
// XNOR-AND with this lane's own bit spread to all 32 bits (0 or ~0).
__device__ inline uint64_t same_bin_lanes(uint32_t bin, bool in, uint32_t nbits) {
  const uint64_t live = __ballot(in);
  uint32_t lo = (uint32_t)live, hi = (uint32_t)(live >> 32);
  for (int bit = 0; bit < 10; ++bit) {
    if ((uint32_t)bit >= nbits) break;
    const uint64_t ones = __ballot((bin >> bit) & 1u);
    const uint32_t mine = (uint32_t)((int32_t)(bin << (31 - bit)) >> 31);
    lo &= ~((uint32_t)ones ^ mine);
    hi &= ~((uint32_t)(ones >> 32) ^ mine);
  }
  return ((uint64_t)hi << 32) | lo;
}

struct SumU32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; }
};
struct SumU64 {
  __device__ uint64_t operator()(uint64_t a, uint64_t b) const { return a + b; }
};
struct SumF64 {
  __device__ double operator()(double a, double b) const { return a + b; }
};
struct MaxI32 {
  __device__ int32_t operator()(int32_t a, int32_t b) const { return a > b ? a : b; }
};
struct MaxU32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};
struct OrU32 {
  __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a | b; }
};

// Exclusive prefix sum over the wave (DPP); `total` receives the wave's sum.
template <class T, class Op>
__device__ inline T wave_excl_scan(T v, Op op, T& total) {
  const T inc = wave_incl_scan(v, op, (T)0);
  total = read_lane(inc, kWaveSize - 1);
  return inc - v;
}
__device__ inline uint32_t wave_excl_sum(uint32_t v, uint32_t& total) {
  return wave_excl_scan(v, SumU32(), total);
}

// IEEE 754-2019 maximum of three floats in one instruction: NaN in any input gives NaN (so a
// running maximum also detects NaN logits), and -0 < +0 (both map to one key later).
__device__ inline float maximum3f(float a, float b, float c) {
  float r;
  asm("v_maximum3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ inline float maximum2f(float a, float b) { return maximum3f(a, b, b); }
struct MaximumF32 {
  __device__ float operator()(float a, float b) const { return maximum2f(a, b); }
};

// Race noise g = -ln(-ln u) in float32 with the hardware log2. Measured over all 2^23 uniforms
// of the race: -ln u has relative error <= 1.7e-7 (also for u next to 1) and g absolute error
// <= 1.7e-6, so a float32 score (x - m)/T + g is within ~3e-6 of exact for every competitive
// candidate (|x - m|/T < 20), far inside kRaceMargin.
__device__ inline float race_noise(float u) {
  const float e = -__builtin_amdgcn_logf(u) * 0.6931471805599453f;
  return -__builtin_amdgcn_logf(e) * 0.6931471805599453f;
}

// Flags and counters between the waves of one workgroup, in LDS. A publish orders every earlier
// LDS write of the wave before the flag (release at workgroup scope); a wait spins with s_sleep
// until the flag reaches a value, then orders the wave's later LDS reads after it. Every flag a
// wave waits on is published unconditionally by waves that never wait on it, so every wait ends;
// each wait is bounded all the same (see lds_wait_at_least), so that a broken publish would end
// the row with an ABORTED status instead of a workgroup that never finishes.
// Counters move in steps of 64: every lane of the wave (always fully active here) adds 1, so
// that no branch on the lane surrounds the atomic (such a branch inside a claim loop has been
// compiled into a loop exit that only lane 0 takes) and the compiler can fold the 64 adds into
// one. Lane 0's previous value, divided by 64, is the number of earlier steps either way.
constexpr uint32_t kStep = kWaveSize;
__device__ inline void lds_publish(uint32_t* flag, uint32_t v) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __hip_atomic_store(flag, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
// One step on a counter after every earlier LDS write of the wave; returns the earlier steps.
__device__ inline uint32_t lds_publish_step(uint32_t* ctr) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return read_lane(old, 0) / kStep;
}
// Claims the next index of a work counter for the whole wave.
__device__ inline uint32_t lds_claim(uint32_t* ctr) {
  const uint32_t old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return read_lane(old, 0) / kStep;
}
// Waits until *flag >= v and returns true; gives up and returns false after `limit` sleeps of
// its own, setting *aborted, or as soon as another wave of the workgroup has set *aborted. A wave
// whose wait gave up skips the rest of its work up to the row's last barrier, where the row gets
// the ABORTED status (fast_row_bf16). One s_sleep(1) is 64 clocks, so the default limit (2^20
// sleeps, tens of milliseconds) is far beyond any wait of a correct row (microseconds).
constexpr uint32_t kDefaultWaitLimit = 1u << 20;
__device__ inline bool lds_wait_at_least(const uint32_t* flag, uint32_t v, uint32_t limit,
                                         uint32_t* aborted) {
  // Lane 0 alone polls: a read by all 64 lanes of one word costs the LDS as much as 64 distinct
  // words, and up to 15 polling waves would otherwise take much of the LDS from the waves that
  // work. The loop's exits test wave-uniform values, so the whole wave leaves together.
  const bool poller = (threadIdx.x & (kWaveSize - 1)) == 0u;
  for (uint32_t spins = 0;; ++spins) {
    uint32_t f = 0u, ab = 0u;
    if (poller) {
      f = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      ab = __hip_atomic_load(aborted, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (uniform_u32(f) >= v) break;
    if (uniform_u32(ab) != 0u) return false;
    if (spins >= limit) {
      __hip_atomic_store(aborted, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      return false;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  return true;
}

__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Capture slot of row b from the first 1024 opt-in entries (e = optin_rows[tid] or INT32_MIN,
// loaded before the row): an entry is valid iff in range and above every earlier entry. Done in
// three steps that share the barriers of the cutoff selection. Marks slot b invalid when it is.
struct SlotScan {
  int32_t e, excl_w;
};
__device__ inline SlotScan slot_step1(int32_t e, FastShared& fs) {
  const uint32_t lane = lane_id(), wid = wave_id();
  const int32_t shifted = dpp_mov<0x138>(INT32_MIN, e);  // wave_shr:1, lane 0 gets INT32_MIN
  const int32_t excl_w = wave_incl_scan(shifted, MaxI32(), INT32_MIN);
  if (lane == kWaveSize - 1) fs.slot_wmax[wid] = excl_w > e ? excl_w : e;
  return {e, excl_w};
}
// After a barrier that follows slot_step1.
__device__ inline void slot_step2(const SampleArgs& a, int64_t b, const SlotScan& sc,
                                  FastShared& fs) {
  const uint32_t tid = threadIdx.x, lane = lane_id(), wid = wave_id();
  int32_t all;
  const int32_t before = waves_prefix(fs.slot_wmax, MaxI32(), INT32_MIN, all);
  const int32_t excl = sc.excl_w > before ? sc.excl_w : before;
  const bool in = (int64_t)tid < a.R;
  const bool valid = in && sc.e >= 0 && (int64_t)sc.e < a.B && sc.e > excl;
  if (in && !valid && (int64_t)tid == b) {
    a.lengths[b] = 0;
    a.selected_logprob[b] = __builtin_nanf("");
  }
  const int32_t hit = wave_reduce(valid && (int64_t)sc.e == b ? (int32_t)tid : -1, MaxI32());
  if (lane == 0) fs.slot_hit[wid] = hit;
}
// After a barrier that follows slot_step2.
__device__ inline int64_t slot_step3(const FastShared& fs) {
  return waves_reduce(fs.slot_hit, MaxI32());
}

// ln(v) for a positive finite double with an absolute error of about 3e-7: the binary exponent
// exactly, the mantissa's logarithm with the hardware log2 in float32.
__device__ inline double ln_fast(double v) {
  int e;
  const double mant = __builtin_frexp(v, &e);  // [0.5, 1)
  return ((double)e + (double)__builtin_amdgcn_logf((float)mant)) * 0.6931471805599453;
}
// The stream's mass sums exp2(x c - R c) as exp2f(fma(x, c, nrc)) with nrc = -R c rounded to
// float, and multiplies by exp2(-nrc - m c) in double afterwards, so that the rounding of nrc
// cancels. That holds while |nrc| <= 2^31: the rounding of R c (up to 2^-25 |R c|, the exponent
// of the maximum's own term) then stays within float exp2's range, and the double R c within
// 2^-22. Rows with top-p and a larger |R / T| (tiny temperatures) go to the general path, whose
// weights use x - m directly (such a row flags every load, or reports an infinite mass, either of
// which sends it there).
constexpr float kMassRefMax = 0x1p31f;

// 2^a for a finite a <= ~0 (every caller passes (x - m) times a positive scale, x <= m), with a
// relative error of about 2e-7 (float32 hardware exp2 on the fractional part, the integer part
// exactly). Arguments below -1100 give 0 anyway (the smallest double is 2^-1074); they are raised
// to -1100 first, so that the integer part always fits an int: converting an out-of-range double
// is undefined, and a float32 row holding a value near 3e38 got infinite weights through it (its
// other values lie ~4e38 below the maximum in log2 units).
__device__ inline double exp2_fast(double a) {
  a = __builtin_fmax(a, -1100.0);
  const double n = __builtin_floor(a);
  return __builtin_ldexp((double)__builtin_amdgcn_exp2f((float)(a - n)), (int)n);
}

// Bin scan by wave 0 alone. Bin d (0 <= d <= dspan) holds the candidates with key kmax - d; they
// were counted by bi = key - theta_key = dspan - d. Only bins d <= dlim are scanned (the bins
// past the min-p cut cannot qualify). Lane l owns the nb consecutive bins from l * nb. Publishes
// the threshold d*, the support size and ln Z_S, and for every support bin its capture base (the
// tokens with larger keys) and (x - m) / T; a logprob is (x - m) / T - ln Z_S.
template <bool NEED_P, int NB, class LY>
__device__ __forceinline__ void bin_scan_wave0(uint32_t kmax, uint32_t dspan, uint32_t dlim, float m,
                                      float T, float c, int32_t k, float p, float mp, double Z,
                                      bool capture, const uint32_t* hcnt, unsigned char* lds,
                                      FastShared& fs) {
  using E = Elem<TSC_DTYPE_BF16>;
  const uint32_t lane = lane_id();
  const uint32_t nb = (dlim + kWaveSize) / kWaveSize;  // 1..NB
  const bool need_m = mp > 0.0f;
  // min-p keeps (x - m) / T >= ln(min_p), i.e. x - m >= T ln(min_p) (x - m is exact in double).
  const double tln_mp = need_m ? (double)T * ln_fast((double)mp) : 0.0;
  // Per bin (all loads first, so that their latencies overlap): value, count after min-p (a
  // per-value predicate, monotone in d), and mass.
  float xs[NB];
  uint32_t cnt[NB];
  double bm[NB];
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const uint32_t d = lane * nb + (uint32_t)t;
    cnt[t] = 0u;
    // An unused slot holds the maximum, so that its mass term cnt * exp2((x - m) c) is 0 * 1:
    // with 0 there, a negative maximum at a low temperature made it 0 * inf = NaN.
    xs[t] = m;
    if ((uint32_t)t < nb && d <= dlim) {
      xs[t] = E::to_float(bits_of_key<E>(kmax - d));
      cnt[t] = hcnt[dspan - d];
    }
  }
  uint32_t lc = 0;
  double lmass = 0.0;
  int32_t low = -1;  // the lane's largest d holding a candidate
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    if (cnt[t] != 0u) low = (int32_t)(lane * nb + (uint32_t)t);
    if (need_m && !(((double)xs[t] - (double)m) >= tln_mp)) cnt[t] = 0u;
    bm[t] = (NEED_P || capture) ? (double)cnt[t] * (double)__builtin_amdgcn_exp2f((xs[t] - m) * c)
                                : 0.0;
    lc += cnt[t];
    lmass += bm[t];
  }
  uint32_t tc;
  double tm;
  uint32_t ec = wave_excl_scan(lc, SumU32(), tc);
  double em = wave_excl_scan(lmass, SumF64(), tm);
  const double pz = (double)p * Z;
  // The largest present d with fewer than k tokens strictly above and, for top_p < 1, mass
  // strictly above <= top_p * Z. Each predicate is monotone in d, so this is the last qualifying
  // bin of the last lane that has one.
  int32_t best = -1;
  uint32_t bL = 0;
  double bZ = 0.0;
  uint32_t* binbase = reinterpret_cast<uint32_t*>(lds + LY::kOffBinBase);
  double* bins = reinterpret_cast<double*>(lds + LY::kOffBinS);
  const double invT = 1.0 / (double)T;
#pragma unroll
  for (int t = 0; t < NB; ++t) {
    const uint32_t d = lane * nb + (uint32_t)t;
    if (cnt[t] != 0u) {
      const bool qual = ec < (uint32_t)k && (!NEED_P || em <= pz);
      if (qual) {
        best = (int32_t)d;
        bL = ec + cnt[t];
        bZ = em + bm[t];
        if (capture) {
          binbase[dspan - d] = ec;
          bins[dspan - d] = ((double)xs[t] - (double)m) * invT;
        }
      }
    }
    ec += cnt[t];
    em += bm[t];
  }
  // d* >= 0 always: bin 0 holds the maximum, which passes every predicate.
  const int32_t dstar = wave_reduce(best, MaxI32());
  const int owner = (int)((uint32_t)dstar / nb);
  const uint32_t L = read_lane(bL, owner);
  const double lnzs = ln_fast(read_lane(bZ, owner));  // logprob = (x - m) / T - ln Z_S
  const int32_t dlow = wave_reduce(low, MaxI32());
  if (lane == 0) {
    fs.decision = kProceed;
    fs.dstar = dstar;
    fs.dlow = dlow;
    fs.L = L;
    fs.lnzs = lnzs;
  }
}

// The last bin d <= dspan (< 1024) whose value passes min-p, by wave 0: the predicate is the scan's
// own and monotone in d, and bin 0 (the maximum) always passes, so one ballot over every 16th bin
// and one over the 16 bins after the last passing one find it.
__device__ inline uint32_t min_p_last_bin(uint32_t kmax, uint32_t dspan, float m, float T, float mp) {
  using E = Elem<TSC_DTYPE_BF16>;
  const uint32_t lane = lane_id();
  const double tln_mp = (double)T * ln_fast((double)mp);
  auto pass = [&](uint32_t d) {
    return d <= dspan && ((double)E::to_float(bits_of_key<E>(kmax - d)) - (double)m) >= tln_mp;
  };
  const uint64_t coarse = __ballot(pass(lane * 16u));
  const uint32_t l0 = 63u - (uint32_t)__builtin_clzll(coarse | 1ull);
  const uint64_t fine = __ballot(lane < 16u && pass(l0 * 16u + lane));
  return l0 * 16u + (63u - (uint32_t)__builtin_clzll(fine | 1ull));
}

// The same for spans of 256 bins and more (bins re-read per pass instead of kept in registers).
template <bool NEED_P, class LY>
__device__ __forceinline__ void bin_scan_wave0_wide(uint32_t kmax, uint32_t dspan, uint32_t dlim,
                                      float m, float T, float c, int32_t k, float p, float mp,
                                      double Z, bool capture, const uint32_t* hcnt,
                                      unsigned char* lds, FastShared& fs) {
  using E = Elem<TSC_DTYPE_BF16>;
  const uint32_t lane = lane_id();
  const uint32_t nb = (dlim + kWaveSize) / kWaveSize;  // 1..16
  const bool need_m = mp > 0.0f;
  // min-p keeps (x - m) / T >= ln(min_p), i.e. x - m >= T ln(min_p) (x - m is exact in double).
  const double tln_mp = need_m ? (double)T * ln_fast((double)mp) : 0.0;
  auto value_of_d = [&](uint32_t d) { return E::to_float(bits_of_key<E>(kmax - d)); };
  // Count and mass of bin d after min-p (a per-value predicate, monotone in d).
  int32_t low = -1;  // the lane's largest d holding a candidate
  auto bin = [&](uint32_t d, uint32_t& bc, double& bm) {
    bc = 0;
    bm = 0.0;
    if (d <= dlim) {
      if (hcnt[dspan - d] != 0u) low = (int32_t)d;
      const float x = value_of_d(d);
      if (!need_m || ((double)x - (double)m) >= tln_mp) {
        bc = hcnt[dspan - d];
        if (NEED_P || capture) bm = (double)bc * (double)__builtin_amdgcn_exp2f((x - m) * c);
      }
    }
  };
  uint32_t lc = 0;
  double lmass = 0.0;
  for (uint32_t t = 0; t < nb; ++t) {
    uint32_t bc;
    double bm;
    bin(lane * nb + t, bc, bm);
    lc += bc;
    lmass += bm;
  }
  uint32_t tc;
  double tm;
  uint32_t ec = wave_excl_scan(lc, SumU32(), tc);
  double em = wave_excl_scan(lmass, SumF64(), tm);
  const double pz = (double)p * Z;
  // The largest present d with fewer than k tokens strictly above and, for top_p < 1, mass
  // strictly above <= top_p * Z. Each predicate is monotone in d, so this is the last qualifying
  // bin of the last lane that has one.
  int32_t best = -1;
  uint32_t bL = 0;
  double bZ = 0.0;
  uint32_t* binbase = reinterpret_cast<uint32_t*>(lds + LY::kOffBinBase);
  double* bins = reinterpret_cast<double*>(lds + LY::kOffBinS);
  const double invT = 1.0 / (double)T;
  for (uint32_t t = 0; t < nb; ++t) {
    const uint32_t d = lane * nb + t;
    uint32_t bc;
    double bm;
    bin(d, bc, bm);
    if (bc != 0u) {
      const bool qual = ec < (uint32_t)k && (!NEED_P || em <= pz);
      if (qual) {
        best = (int32_t)d;
        bL = ec + bc;
        bZ = em + bm;
        if (capture) {
          binbase[dspan - d] = ec;
          bins[dspan - d] = ((double)value_of_d(d) - (double)m) * invT;
        }
      }
    }
    ec += bc;
    em += bm;
  }
  // d* >= 0 always: bin 0 holds the maximum, which passes every predicate.
  const int32_t dstar = wave_reduce(best, MaxI32());
  const int owner = (int)((uint32_t)dstar / nb);
  const uint32_t L = read_lane(bL, owner);
  const double lnzs = ln_fast(read_lane(bZ, owner));  // logprob = (x - m) / T - ln Z_S
  const int32_t dlow = wave_reduce(low, MaxI32());
  if (lane == 0) {
    fs.decision = kProceed;
    fs.dstar = dstar;
    fs.dlow = dlow;
    fs.L = L;
    fs.lnzs = lnzs;
  }
}


// Sets the bitmask bit of every survivor (value >= x_cut) of one wave's candidate list, whose
// ids ascend, in a mask row zeroed beforehand. 64 candidates at a time: the lanes whose ids share
// a 32-bit word form a run, a segmented OR over the runs (DPP steps) gathers each run's bits into
// its last lane, and every word is written once. The group's last run is carried into the next
// group, so that a word the two share is still written once. A plain store suffices for every
// word but the list's first and last, which the neighbouring waves' lists may share and which
// take an atomic OR. Atomic ORs on words that plain stores also wrote were slow: one atomic per
// survivor took the k = 8192 workload with bitmasks to 87 us (47 now), and the B=256, V=151936,
// k=1024 rows captured at W = 512 to 27.7 us (25.6 now).
__device__ inline void support_bits_of_list(const uint32_t* cand, uint32_t n, float x_cut,
                                            uint32_t id0, uint32_t* brow) {
  const uint32_t lane = lane_id();
  if (n == 0u) return;
  constexpr uint32_t kNone = 0xFFFFFFFFu;
  const uint32_t list_first = (id0 + (cand[0] & 0x3FFFu)) >> 5;
  const uint32_t list_last = (id0 + (cand[n - 1u] & 0x3FFFu)) >> 5;
  auto put = [&](uint32_t w, uint32_t b) {
    if (b == 0u) return;
    if (w == list_first || w == list_last)
      atomicOr(brow + w, b);
    else
      brow[w] = b;
  };
  uint32_t carry_w = kNone, carry_b = 0u;  // the previous group's last run, not yet written
  for (uint32_t base = 0; base < n; base += kWaveSize) {  // uniform: every lane takes part
    const uint32_t i = base + lane;
    const bool valid = i < n;
    const uint32_t wd = valid ? cand[i] : 0u;
    const uint32_t id = id0 + (wd & 0x3FFFu);
    const uint32_t widx = valid ? id >> 5 : kNone;
    uint32_t bits = valid && __uint_as_float(wd & 0xFFFF0000u) >= x_cut ? 1u << (id & 31u) : 0u;
    // Segmented inclusive OR (the steps of the wave scan; a source lane of the same word lies in
    // the same run): each run's last lane ends up with the run's bits.
    auto step = [&](auto mv) {
      const uint32_t ow = mv(kNone, widx), ob = mv(0u, bits);
      if (ow == widx) bits |= ob;
    };
    step([](uint32_t o, uint32_t v) { return dpp_mov<dpp::kRowShr1>(o, v); });
    step([](uint32_t o, uint32_t v) { return dpp_mov<dpp::kRowShr2>(o, v); });
    step([](uint32_t o, uint32_t v) { return dpp_mov<dpp::kRowShr4>(o, v); });
    step([](uint32_t o, uint32_t v) { return dpp_mov<dpp::kRowShr8>(o, v); });
    step([](uint32_t o, uint32_t v) { return dpp_mov<dpp::kRowBcast15, 0xA>(o, v); });
    step([](uint32_t o, uint32_t v) { return dpp_mov<dpp::kRowBcast31, 0xC>(o, v); });
    const uint32_t next = __shfl_down(widx, 1, kWaveSize);
    const uint32_t last = (n - base < (uint32_t)kWaveSize ? n - base : (uint32_t)kWaveSize) - 1u;
    const bool tail = valid && (lane == last || next != widx);
    const uint32_t g_first = read_lane(widx, 0), g_last = read_lane(widx, (int)last);
    if (carry_w == g_first) {
      if (tail && widx == g_first) bits |= carry_b;  // the carried run continues here
    } else if (carry_w != kNone && lane == 0) {
      put(carry_w, carry_b);
    }
    carry_w = g_last;
    carry_b = read_lane(bits, (int)last);
    if (tail && widx != g_last) put(widx, bits);
  }
  if (lane == 0) put(carry_w, carry_b);
}

template <bool COMPACT> struct LayoutOf { using type = LayoutStash; };
template <> struct LayoutOf<true> { using type = LayoutCompact; };

// Fast path of one bfloat16 row. Returns false (having written no row output) when the row must
// go through the general path instead; `slot` is then already set.
template <bool NEED_P, bool COMPACT, int LOADS, bool BITS>
__device__ __forceinline__ bool fast_row_bf16(const SampleArgs& a, int64_t b, int64_t& slot,
                                              float T, int32_t k, int32_t kv, float p, float mp,
                                              uint64_t seed, uint64_t pos, unsigned char* lds,
                                              FastShared& fs) {
  using E = Elem<TSC_DTYPE_BF16>;
  using LY = typename LayoutOf<COMPACT>::type;
  const uint32_t tid = threadIdx.x, lane = lane_id(), wid = wave_id();
  const uint16_t* row = reinterpret_cast<const uint16_t*>(a.logits) + b * a.ld;
  const uint4* rowv = reinterpret_cast<const uint4*>(row);
  const int64_t V = a.V;
  const uint32_t nch = (uint32_t)(V / 8);
  const uint32_t cw = (nch + kWaves - 1) / kWaves;        // chunks per wave segment
  const uint32_t seg0 = wid * cw;
  const uint32_t seg1 = seg0 + cw < nch ? seg0 + cw : nch;
  const uint32_t nseg = seg1 - seg0;                      // chunks in this wave's segment
  const uint32_t id0 = seg0 * 8u;                         // first token id of the segment

  // Rank of theta among the lane maxima of the first kSampleLoads loads of every segment (up to
  // 1024 kSampleLoads chunk maxima). A chunk's maximum exceeds the k-th largest value with
  // probability at most p_k = 1 - (1 - k/V)^8, so the number of sampled maxima above that value
  // is at most binomial with mean mu = n p_k and variance n p_k (1 - p_k). theta is the sampled
  // maximum of rank mu + 5 sd + 6: it lies above the k-th value (the row then leaves for the
  // general path) with probability of the order of 1e-7 or below for independent logits, from
  // a Poisson-like count at small mu to a normal tail at large mu. Rows of the short form sample
  // four loads, which halves the variance and so cuts the candidates of k = 1024 rows
  // (V = 151936) by ~15%; rows of the long form sample two, because the later exchange that four
  // loads need slowed their stream by ~0.8 us (B=1024, V=262144), more than the smaller tail
  // saved.
  constexpr int kSampleLoads = LOADS == kShortLoads ? 4 : 2;
  constexpr int kSamples = kSampleLoads * kThreads;
  uint32_t theta_rank;
  {
    const float n = (float)(nch < (uint32_t)kSamples ? nch : (uint32_t)kSamples);
    const float t = 1.0f - fminf(1.0f, (float)kv / (float)V);
    const float t2 = t * t, t4 = t2 * t2;
    const float pk = 1.0f - t4 * t4;
    const float mu = n * pk;
    const float rr = ceilf(mu + 5.0f * sqrtf(mu * (1.0f - pk)) + 6.0f);
    theta_rank = (uint32_t)(rr < 1.0f ? 1.0f : (rr > (float)kSamples ? (float)kSamples : rr));
  }

  // Wave priorities: streaming waves issue first (priority 3). A wave whose stream has ended
  // works on at a priority set by how late it ended, so that the post-stream work of early waves
  // fills the issue slots the streaming waves leave idle instead of delaying them (the
  // instruction arbiter otherwise favours the oldest wave, which also ends first).
  __builtin_amdgcn_s_setprio(3);

  // ---- 1. Loads: the opt-in entry first (loads complete in issue order, so waiting for it never
  // waits for row data), then a shallow pipeline over the wave's segment: two loads at first, so
  // that every wave's first load lands within ~2 us, then kLoadsAhead.
  const int32_t opt_e = (a.R <= kThreads && (int64_t)tid < a.R) ? a.optin_rows[tid] : INT32_MIN;
  // Buffer loads: the wave's segment is one scalar resource descriptor (loads past its end return
  // zero and are replaced below), one shared VGPR offset, and a scalar offset per load.
  uint4 r[LOADS];
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint4*>(rowv + seg0), (short)0, (int)(nseg * 16u), 0x00020000);
  const int voff = (int)(lane * 16u);
  // Non-temporal (cache policy NT): the row is read once, and streaming it past the caches
  // measured ~10% more bandwidth than default loads for this one-row-per-workgroup shape.
  auto issue = [&](int j) {
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, j * kWaveSize * 16, 2);
    r[j] = make_uint4(v.x, v.y, v.z, v.w);
  };
#pragma unroll
  for (int j = 0; j < kLoadsFirst; ++j) issue(j);
  // Keep the loads here: nothing orders global loads against the LDS-only barriers that follow,
  // and the scheduler would otherwise sink them towards their first use.
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

  uint32_t* hcnt = reinterpret_cast<uint32_t*>(lds + LY::kOffCnt);
  hcnt[tid] = 0u;  // published by the first exchange below
  if (tid < (uint32_t)kThetaBins / 2) fs.theta_hist[tid] = 0u;
  if (tid == 0) {
    fs.ndone = 0u;
    fs.aborted = 0u;
    fs.scan_ready = 0u;
    fs.prefix_done = 0u;
    fs.job_next = 0u;
    fs.ready = 0u;
    fs.cap_next = 0u;
    fs.staged = 0u;
    fs.copy_next = 0u;
    fs.bits_next = 0u;
  }
  reinterpret_cast<uint64_t*>(lds + LY::kOffBinBest)[tid] = 0ull;

  // Lanes past the segment's end read zeros: only loads that reach the end need the test.
  const uint32_t nfull = uniform_u32(nseg / kWaveSize);  // loads wholly inside the segment
  auto mask_tail = [&](int j) {
    if ((uint32_t)j >= nfull) {  // wave-uniform: a scalar branch, no vector work on full loads
      if ((uint32_t)j * kWaveSize + lane >= nseg)
        r[j] = make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
    }
  };
  auto unpack = [](const uint4& q, float (&f)[8]) {
    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16_lo(w4[e]);
      f[2 * e + 1] = bf16_hi(w4[e]);
    }
  };
  auto load_max = [](const float (&f)[8]) {
    const float a0 = maximum3f(f[0], f[1], f[2]);
    const float a1 = maximum3f(f[3], f[4], f[5]);
    return maximum3f(a0, a1, maximum2f(f[6], f[7]));
  };

  // ---- 2. Stream: max, mass, cutoff, stash ---------------------------------------------------
  const float c = 1.4426950408889634f / T;  // log2(e) / T
  float nrc = 0.0f;               // -R * c, R the reference of the mass (set after exchange 1)
  float m_l = -__builtin_inff();  // lane maximum (NaN if the lane saw a NaN)
  float s_a = 0.0f, s_b = 0.0f;   // lane mass: sums of exp2(x * c - R * c), two chains
  auto add_mass = [&](const float (&f)[8]) {
    if constexpr (NEED_P) {
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        s_a += __builtin_amdgcn_exp2f(__builtin_fmaf(f[e], c, nrc));
        s_b += __builtin_amdgcn_exp2f(__builtin_fmaf(f[e + 1], c, nrc));
      }
    }
  };
  uint32_t wcnt = 0;   // wave's flagged loads, or its candidates (compaction; wave-uniform)
  uint32_t wfill = 0;  // stash slots written: wcnt until a load no longer fits
  uint4* stash = reinterpret_cast<uint4*>(lds + LayoutStash::kOffStash) + wid * kStashPerWave;
  uint32_t* stash_ch =
      reinterpret_cast<uint32_t*>(lds + LayoutStash::kOffStashCh) + wid * kStashPerWave;
  float theta = __builtin_inff();
  // Compaction: the load's values >= theta are appended to the wave's list in id order (lane
  // counts, one DPP scan for the slots); a wave-load without any is skipped. Candidates past
  // the capacity are counted, not written, and the row falls back.
  auto compact_load = [&](int j, const uint4& q) {
    // Candidate word: bf16 bits << 16 | offset of the token in the segment (< 2^14). Elements
    // that are not candidates go to a dummy slot of this lane (branch-free scatter).
    uint32_t* cand = reinterpret_cast<uint32_t*>(lds + LY::kOffCand) + wid * LY::kCandCap;
    uint32_t* dummy = reinterpret_cast<uint32_t*>(lds + LY::kOffDummy) + lane;
    // theta is finite whenever the row can be served here; clamping it keeps -inf out.
    const float th = theta > -3.4028234663852886e38f ? theta : -3.4028234663852886e38f;
    const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
    const uint32_t off = ((uint32_t)j * kWaveSize + lane) * 8u;
    uint32_t words[8];
    bool isc[8];
    uint32_t n = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t hi = (e & 1) ? (w4[e >> 1] & 0xFFFF0000u) : (w4[e >> 1] << 16);
      isc[e] = __uint_as_float(hi) >= th;  // -0 ties +0; NaN fails
      words[e] = hi | (off + (uint32_t)e);
      n += isc[e];
    }
    if (__ballot(n != 0u) == 0ull) return;
    uint32_t total;
    uint32_t at = wcnt + wave_excl_sum(n, total);
    if (wcnt + total <= (uint32_t)LY::kCandCap) {  // wave-uniform: no capacity test per element
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t* dst = isc[e] ? cand + at : dummy;
        *dst = words[e];
        at += isc[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t* dst = (isc[e] && at < (uint32_t)LY::kCandCap) ? cand + at : dummy;
        *dst = words[e];
        at += isc[e];
      }
    }
    wcnt += total;
  };
  uint16_t* spill = reinterpret_cast<uint16_t*>(lds + LayoutStash::kOffSpill) + wid * kSpillPerWave;
  auto stash_load = [&](int j, const uint4& q, bool flag) {
    const uint64_t mask = __ballot(flag);
    const uint32_t n = (uint32_t)__popcll(mask);
    // Capacity is checked per load for the whole wave (scalar), so the flagged lanes only
    // compute their slot. A load that no longer fits the stash (and every later one: the count
    // only grows) keeps just its chunk index, and is read again after the stream; past that
    // list too, the row falls back.
    if (n != 0u) {
      const uint32_t chunk = (uint32_t)j * kWaveSize + lane;  // chunk within the segment
      if (wcnt + n <= (uint32_t)kStashPerWave) {
        if (flag) {
          const uint32_t at = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                        __builtin_amdgcn_mbcnt_lo((uint32_t)mask, wcnt));
          stash[at] = q;
          stash_ch[at] = chunk;
        }
        wfill = wcnt + n;
      } else if (wcnt - wfill + n <= (uint32_t)kSpillPerWave) {
        if (flag) {
          const uint32_t at = __builtin_amdgcn_mbcnt_hi(
              (uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, wcnt - wfill));
          spill[at] = (uint16_t)chunk;
        }
      }
    }
    wcnt += n;
  };
  // Keep each load's work at its own step: without this the compiler may sink the exp chain
  // (which only feeds the final sum) past the loop and keep every load's data alive.
  auto pin = [&]() { asm volatile("" : "+v"(s_a), "+v"(s_b), "+v"(m_l)); };

  // Step 0, exchange 1: wave maxima of the first-load lane maxima; slot scan, step 1.
  float f[8];
  mask_tail(0);
  unpack(r[0], f);
  const float lm0 = load_max(f);
  m_l = maximum2f(m_l, lm0);
  // The first load has landed: only now deepen the pipeline (issuing earlier would delay it).
  asm volatile("" ::"v"(lm0));
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int jj = kLoadsFirst; jj <= kLoadsAhead && jj < LOADS; ++jj) issue(jj);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  const uint32_t key0 = key_of<E>(__float_as_uint(lm0) >> 16);
  {
    const uint32_t wk = wave_reduce(key0, MaxU32());
    if (lane == 0) fs.kmax0_w[wid] = wk;
  }
  const SlotScan sscan = slot_step1(opt_e, fs);
  lds_barrier();
  // Step 1: the mass reference R = the first loads' maximum; the first two loads' maxima enter
  // the histogram of the distances to it.
  const uint32_t kmax0 = waves_reduce(fs.kmax0_w, MaxU32());
  {
    const float R = E::to_float(bits_of_key<E>(kmax0));
    // A non-finite sample maximum (all -inf, or +inf/NaN: the row is then nonfinite anyway)
    // takes R = 0; a mass that overflows sends the row to the general path.
    nrc = uniform_f32(__builtin_isfinite(R) ? -R * c : 0.0f);
  }
  add_mass(f);
  issue(kLoadsAhead + 1);
  mask_tail(1);
  unpack(r[1], f);
  const float lm1 = load_max(f);
  m_l = maximum2f(m_l, lm1);
  add_mass(f);
  pin();
  {
    // Distances below the first loads' maximum (the second load's maximum may lie above it: then
    // distance 0); keys below 0x80 are -inf or NaN and are not counted.
    const uint32_t key1 = key_of<E>(__float_as_uint(lm1) >> 16);
    const uint32_t dist0 = kmax0 - key0;
    const uint32_t dist1 = key1 >= kmax0 ? 0u : kmax0 - key1;
    if (dist0 < (uint32_t)kThetaBins && (key0 >> 7) != 0u)
      atomicAdd(&fs.theta_hist[dist0 >> 1], 1u << (16u * (dist0 & 1u)));
    if (dist1 < (uint32_t)kThetaBins && (key1 >> 7) != 0u)
      atomicAdd(&fs.theta_hist[dist1 >> 1], 1u << (16u * (dist1 & 1u)));
  }
  // Lane maxima of the sampled loads (loads 0 .. kSampleLoads), for their stash decisions.
  float lmx[kSampleLoads + 1];
  lmx[0] = lm0;
  lmx[1] = lm1;
  auto hist_add = [&](float lmv) {
    const uint32_t kx = key_of<E>(__float_as_uint(lmv) >> 16);
    const uint32_t dx = kx >= kmax0 ? 0u : kmax0 - kx;
    if (dx < (uint32_t)kThetaBins && (kx >> 7) != 0u)
      atomicAdd(&fs.theta_hist[dx >> 1], 1u << (16u * (dx & 1u)));
  };
  auto step = [&](int j) {  // load j: maximum and mass
    issue(kLoadsAhead + j);
    mask_tail(j);
    unpack(r[j], f);
    lmx[j] = load_max(f);
    m_l = maximum2f(m_l, lmx[j]);
    add_mass(f);
    pin();
  };
  // Short form, steps 2 and 3: the next two loads' maxima join the histogram.
  if constexpr (kSampleLoads == 4) {
    step(2);
    hist_add(lmx[2]);
    step(3);
    hist_add(lmx[3]);
  }
  // Exchange 2 (every sampled maximum is in the histogram) and slot step 2.
  if (a.R <= kThreads) slot_step2(a, b, sscan, fs);
  lds_barrier();
  // Next step: every wave finds the smallest distance whose cumulative count reaches the rank
  // (when fewer maxima are within reach, the deepest reachable key); the same scan in each wave
  // saves an exchange.
  step(kSampleLoads);
  uint32_t theta_key;
  {
    // At most 4096 samples, so a u16 count never carries into its neighbour.
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
    theta_key = uniform_u32(kmax0 > dsel ? kmax0 - dsel : 0u);
  }
  // Min-p floor. min-p keeps x - m >= T ln(min_p), and the row maximum m is at least the largest
  // sampled value r0, so no token below r0 + T ln(min_p) is in the support: theta rises to that
  // floor when it is higher (heavy-headed rows keep a handful of candidates instead of thousands
  // chosen for k). The floor sits 2^-16 of its terms below the float computation, far more than
  // the rounding of that computation and the error of the scan's ln(min_p), so that every token
  // below theta fails the scan's own min-p test, which the decision after the scan checks.
  if (mp > 0.0f) {
    const float r0 = E::to_float(bits_of_key<E>(kmax0));
    const float lnmp = __logf(mp);
    const float g = r0 + T * lnmp;
    const float floor_v = g - (__builtin_fabsf(r0) + T * __builtin_fabsf(lnmp) + T) * 0x1p-16f;
    // (NaN or infinite terms leave theta as it is.)
    if (__builtin_isfinite(floor_v)) {
      // The largest bfloat16 value <= floor_v: truncation, one key lower where truncating a
      // negative value rounded it up.
      const uint32_t fb = __float_as_uint(floor_v) >> 16;
      uint32_t fk = key_of<E>(fb);
      if (E::to_float(fb) > floor_v) fk -= 1u;
      theta_key = uniform_u32(fk > theta_key ? fk : theta_key);
    }
  }
  theta = E::to_float(bits_of_key<E>(theta_key));
  slot = a.R <= kThreads ? slot_step3(fs) : find_capture_slot(a, b, fs.red);
#pragma unroll
  for (int j = 0; j <= kSampleLoads; ++j) {
    if constexpr (COMPACT) compact_load(j, r[j]);
    else stash_load(j, r[j], lmx[j] >= theta);
  }
  // From here on, for top_p < 1, a load is stashed when the sum of its weights reaches the
  // weight of theta (any element >= theta implies it; the small slack covers exp2 rounding), so
  // the load's maximum is not needed: the row maximum is the largest candidate, and a NaN logit
  // shows up in the mass.
  // (A theta weight below 2^-100 would flag every load: the stash overflows and the row falls
  // back, which happens only for extreme spreads of the logits at low temperature.)
  // (A reference past kMassRefMax flags every load: the stash overflows, and the row leaves for
  // the general path through the overflow test.)
  const float wth = __builtin_fabsf(nrc) <= kMassRefMax
                        ? 0.99999f * __builtin_amdgcn_exp2f(__builtin_fmaf(theta, c, nrc))
                        : 0.0f;
  // Race draws of 128 candidates from `base` of this wave's list (two Philox chains per lane).
  // Each candidate's uniform is kept per bin as max(u numerator << 32 | ~id) (see the pick).
  uint64_t* binbest = reinterpret_cast<uint64_t*>(lds + LY::kOffBinBest);
  const uint32_t* cand_own = reinterpret_cast<const uint32_t*>(lds + LY::kOffCand) + wid * LY::kCandCap;
  auto draw_job = [&](uint32_t base, uint32_t lim) {
    const uint32_t i0 = base + lane, i1 = i0 + kWaveSize;
    const bool v0 = i0 < lim, v1 = i1 < lim;
    const uint32_t wd0 = v0 ? cand_own[i0] : 0u, wd1 = v1 ? cand_own[i1] : 0u;
    const uint32_t id0w = id0 + (wd0 & 0x3FFFu), id1w = id0 + (wd1 & 0x3FFFu);
    const uint32_t r0 = race_word(id0w, seed, pos);
    const uint32_t r1 = race_word(id1w, seed, pos);
    const uint32_t bi0 = key_of<E>(wd0 >> 16) - theta_key, bi1 = key_of<E>(wd1 >> 16) - theta_key;
    if (v0 && bi0 < (uint32_t)kDBins)
      atomicMax(reinterpret_cast<unsigned long long*>(&binbest[bi0]),
                ((unsigned long long)(2u * (r0 >> 9) + 1u) << 32) | (unsigned long long)(~id0w));
    if (v1 && bi1 < (uint32_t)kDBins)
      atomicMax(reinterpret_cast<unsigned long long*>(&binbest[bi1]),
                ((unsigned long long)(2u * (r1 >> 9) + 1u) << 32) | (unsigned long long)(~id1w));
  };
#pragma unroll
  for (int j = kSampleLoads + 1; j < LOADS; ++j) {
    // Every step issues its load unconditionally (loads past the segment read zeros through the
    // buffer descriptor, with no memory traffic): a conditional issue makes the compiler's wait
    // counts conservative (vmcnt(0) at every step), which serialises the load pipeline.
    if (j + kLoadsAhead < LOADS) issue(j + kLoadsAhead);
    mask_tail(j);
    unpack(r[j], f);
    bool flag;
    if constexpr (NEED_P) {
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[i], c, nrc));
      const float ls = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
      if (j & 1) s_b += ls; else s_a += ls;
      flag = ls >= wth;
    }
    if constexpr (!NEED_P || COMPACT) {
      const float lm = load_max(f);
      m_l = maximum2f(m_l, lm);
      if constexpr (!NEED_P) flag = lm >= theta;
    }
    pin();
    if constexpr (COMPACT) compact_load(j, r[j]);
    else stash_load(j, r[j], flag);
  }

  // ---- 3. Per wave, as soon as its segment is done: partials, expansion, counts ---------------
  uint32_t order;  // 0 for the first wave whose stream ended, 15 for the last
  {
    uint32_t o = 0;
    if (lane == 0) o = atomicAdd(&fs.ndone, 1u);
    order = uniform_u32(read_lane(o, 0));
  }
  if (order < (uint32_t)kWaves - 8) __builtin_amdgcn_s_setprio(0);
  else if (order < (uint32_t)kWaves - 4) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(2);
  {
    double wz = 0.0;
    if constexpr (NEED_P) wz = wave_reduce((double)(s_a + s_b), SumF64());
    if (lane == 0) {
      fs.wave_z[wid] = wz;
      fs.wave_stash[wid] = COMPACT ? 0u : wcnt - wfill;  // loads past the stash
    }
  }
  // Candidate word: bf16 bits << 16 | offset of the token in the segment (< 2^14), in id order.
  uint32_t* cand = reinterpret_cast<uint32_t*>(lds + LY::kOffCand) + wid * LY::kCandCap;
  // theta is finite whenever the row can be served here; clamping it keeps -inf out.
  const float th = theta > -3.4028234663852886e38f ? theta : -3.4028234663852886e38f;
  uint32_t ncand = 0;            // wave-uniform
  float xcand = -__builtin_inff();  // lane maximum of the candidates
  if constexpr (COMPACT) {
    ncand = wcnt;
    xcand = m_l >= th ? m_l : -__builtin_inff();  // the lane maximum is a candidate iff >= theta
  } else {
    // Stash expansion: candidate words of the stashed loads, then of the loads past the stash
    // (read again now), in id order. Lanes without a load hold -inf, which no candidate is.
    uint32_t* const dummy = reinterpret_cast<uint32_t*>(lds + LY::kOffDummy) + lane;
    auto expand_chunk = [&](const uint4& q, uint32_t off) {
      const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
      uint32_t words[8];
      float xc[8];
      uint32_t cm = 0;  // bit e: element e is a candidate
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t hi = (e & 1) ? (w4[e >> 1] & 0xFFFF0000u) : (w4[e >> 1] << 16);
        const bool isc = __uint_as_float(hi) >= th;  // -0 ties +0; NaN fails
        xc[e] = isc ? __uint_as_float(hi) : -__builtin_inff();
        words[e] = hi | (off + (uint32_t)e);
        cm |= (uint32_t)isc << e;
      }
      xcand = maximum3f(xcand, maximum3f(xc[0], xc[1], xc[2]), maximum3f(xc[3], xc[4], xc[5]));
      xcand = maximum3f(xcand, xc[6], xc[7]);
      uint32_t total;
      const uint32_t at = ncand + wave_excl_sum((uint32_t)__popc(cm), total);
      // Element e goes to at + (candidates before it in the lane), a bit count each (no chain
      // through the elements); the others go to the lane's dummy slot, so that no store needs
      // its own execution mask. Past the capacity nothing is written (the row falls back).
      if (ncand + total <= (uint32_t)LY::kCandCap) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint32_t* dst = ((cm >> e) & 1u) ? cand + (at + (uint32_t)__popc(cm & ((1u << e) - 1u))) : dummy;
          *dst = words[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t pos = at + (uint32_t)__popc(cm & ((1u << e) - 1u));
          uint32_t* dst = ((cm >> e) & 1u) && pos < (uint32_t)LY::kCandCap ? cand + pos : dummy;
          *dst = words[e];
        }
      }
      ncand += total;
    };
    const uint4 kNone = make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
    constexpr int kChunks = kStashPerWave / kWaveSize;
    // Loads past the stash (when the list overflowed, the row falls back: none are read). The
    // first batch is read before the stash is expanded, so that its latency overlaps that work.
    const uint32_t nspill = wcnt - wfill <= (uint32_t)kSpillPerWave ? wcnt - wfill : 0u;
    uint4 sq[kChunks];
    uint32_t so[kChunks];
    auto read_spills = [&](uint32_t base) {
#pragma unroll
      for (int ch = 0; ch < kChunks; ++ch) {
        const uint32_t i = base + (uint32_t)ch * kWaveSize + lane;
        sq[ch] = kNone;
        so[ch] = 0u;
        if (base + (uint32_t)ch * kWaveSize < nspill && i < nspill) {
          // (A lane past the segment's end holds -inf in the stream; its chunk is not read.)
          const uint32_t chunk = spill[i];
          if (chunk < nseg) {
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(chunk * 16u), 0, 0);
            sq[ch] = make_uint4(v.x, v.y, v.z, v.w);
            so[ch] = chunk * 8u;
          }
        }
      }
    };
    if (nspill > 0u) read_spills(0u);
    const uint32_t nstash = wfill;  // never slots that were not written in this row
    // All stash reads first (at most 4 chunks of 64 loads), so that their latencies overlap.
    uint4 qs[kChunks];
    uint32_t offs[kChunks];
#pragma unroll
    for (int ch = 0; ch < kChunks; ++ch) {
      const uint32_t i = (uint32_t)ch * kWaveSize + lane;
      qs[ch] = kNone;
      offs[ch] = 0u;
      if ((uint32_t)ch * kWaveSize < nstash && i < nstash) {
        qs[ch] = stash[i];
        offs[ch] = stash_ch[i] * 8u;
      }
    }
#pragma unroll
    for (int ch = 0; ch < kChunks; ++ch) {
      if ((uint32_t)ch * kWaveSize >= nstash) break;
      expand_chunk(qs[ch], offs[ch]);
    }
    for (uint32_t base = 0; base < nspill; base += kChunks * kWaveSize) {
      if (base > 0u) read_spills(base);
#pragma unroll
      for (int ch = 0; ch < kChunks; ++ch) {
        if (base + (uint32_t)ch * kWaveSize >= nspill) break;
        expand_chunk(sq[ch], so[ch]);
      }
    }
  }
  // The wave's count table (in stash mode its stash slice, free now).
  uint16_t* bincnt = reinterpret_cast<uint16_t*>(lds + LY::kOffTables + wid * LY::kTableStride);
  for (uint32_t i = lane; i < (uint32_t)kTableBytes / 16; i += kWaveSize)
    reinterpret_cast<uint4*>(bincnt)[i] = make_uint4(0u, 0u, 0u, 0u);
  const uint32_t nc_here = ncand < (uint32_t)LY::kCandCap ? ncand : (uint32_t)LY::kCandCap;
  // Maximum: for top_p < 1 the largest candidate (the row maximum is >= theta, so it is one);
  // otherwise the running maximum of the stream (which also carries NaN).
  const float wxc = wave_reduce(xcand, MaximumF32());
  {
    float wm = wxc;
    if constexpr (!NEED_P) wm = wave_reduce(m_l, MaximumF32());
    if (lane == 0) fs.wave_m[wid] = wm;
  }
  const uint32_t bmax = wxc > -__builtin_inff() ? key_of<E>(__float_as_uint(wxc) >> 16) - theta_key : 0u;
  // Compaction mode: the rank of candidate 64 c + lane among the wave's earlier candidates of its
  // bin, two 16-bit ranks per register, kept until the capture (a bin is wholly in the support or
  // wholly out, so ranks among all candidates are ranks among the survivors).
  constexpr int kRankRegs = COMPACT ? LY::kCandCap / kWaveSize / 2 : 1;
  uint32_t crank[kRankRegs];
  if constexpr (COMPACT) {
    // The bin's count in earlier chunks (this wave's own table: plain reads and writes) plus the
    // lanes of its bin below it in this chunk: a 64-bit lane mask per bin that every lane ORs its
    // bit into (the wave's 2 KB slice of the stage, unused until the capture), or, when the wave's
    // bins reach beyond the mask table, ballots over the bits of the bin. The bin's first lane
    // stores the new count, clears the mask and adds the chunk's count to the row histogram.
    uint64_t* binmask = reinterpret_cast<uint64_t*>(lds + LY::kOffStage) + wid * kMaskBins;
    static_assert(kWaves * kMaskBins * 8 <= LY::kStageCap * 4, "lane masks fit the stage");
    const bool by_mask = bmax < (uint32_t)kMaskBins;
    if (by_mask)
      for (uint32_t i = lane; i < (uint32_t)kMaskBins; i += kWaveSize) binmask[i] = 0ull;
    const uint32_t nbits_w = bmax < (uint32_t)kDBins ? 32u - (uint32_t)__builtin_clz(bmax | 1u) : 10u;
    // One LDS round trip per chunk: the next chunk's words are read ahead, and the mask and the
    // count are read together.
    uint32_t wd_next = lane < nc_here ? cand[lane] : 0xFF800000u;
#pragma unroll
    for (int cc = 0; cc < 2 * kRankRegs; ++cc) {
      uint32_t r = 0u;
      if ((uint32_t)cc * kWaveSize < nc_here) {
        const uint32_t i = (uint32_t)cc * kWaveSize + lane;
        const uint32_t wd = wd_next;
        if (cc + 1 < 2 * kRankRegs) {
          const uint32_t in_ = i + kWaveSize;
          wd_next = in_ < nc_here ? cand[in_] : 0xFF800000u;
        }
        const uint32_t bi = key_of<E>(wd >> 16) - theta_key;
        const bool in = i < nc_here && bi < (uint32_t)kDBins;  // wider spans fall back (span test)
        uint64_t same;
        uint32_t c0 = 0u;
        if (by_mask) {
          if (in) atomicOr(reinterpret_cast<unsigned long long*>(&binmask[bi]), 1ull << lane);
          same = in ? binmask[bi] : 0ull;
          c0 = in ? bincnt[bi] : 0u;
        } else {
          same = same_bin_lanes(bi, in, nbits_w);
          c0 = in ? bincnt[bi] : 0u;
        }
        if (in) {
          r = c0 + mbcnt(same);
          if (lane == (uint32_t)__builtin_ctzll(same)) {
            const uint32_t cnt = (uint32_t)__popcll(same);
            bincnt[bi] = (uint16_t)(c0 + cnt);
            if (by_mask) binmask[bi] = 0ull;
            atomicAdd(&hcnt[bi], cnt);
          }
        }
      }
      if (cc & 1) crank[cc >> 1] |= r << 16;
      else crank[cc >> 1] = r;
    }
  } else {
    // Rank of each candidate among the wave's earlier candidates of its bin: the bin's count in
    // earlier chunks (this wave's own table, so plain reads and writes) plus the lanes of its
    // bin below it in this chunk. Those lanes come from a 64-bit mask per bin that every lane
    // ORs its bit into, or, when the wave's bins reach beyond the mask table, from ballots over
    // the bits of the bin. The bin's first lane stores the new count and adds the chunk's count
    // to the row histogram.
    uint64_t* binmask = reinterpret_cast<uint64_t*>(bincnt + kDBins);
    uint16_t* rankw = reinterpret_cast<uint16_t*>(lds + LayoutStash::kOffRank) + wid * LY::kCandCap;
    for (uint32_t i = lane; i < (uint32_t)kMaskBins; i += kWaveSize) binmask[i] = 0ull;
    const bool by_mask = bmax < (uint32_t)kMaskBins;
    for (uint32_t base = 0; base < nc_here; base += kWaveSize) {
      const uint32_t i = base + lane;
      const uint32_t wd = i < nc_here ? cand[i] : 0xFF800000u;
      const uint32_t bi = key_of<E>(wd >> 16) - theta_key;
      const bool in = i < nc_here && bi < (uint32_t)kDBins;  // wider spans fall back (span test)
      uint64_t same;
      if (by_mask) {
        if (in) atomicOr(reinterpret_cast<unsigned long long*>(&binmask[bi]), 1ull << lane);
        same = in ? binmask[bi] : 0ull;
      } else {
        same = same_bin_lanes(bi, in, 10u);
      }
      if (in) {
        const uint32_t c0 = bincnt[bi];
        rankw[i] = (uint16_t)(c0 + mbcnt(same));
        if (lane == (uint32_t)__builtin_ctzll(same)) {
          const uint32_t cnt = (uint32_t)__popcll(same);
          bincnt[bi] = (uint16_t)(c0 + cnt);
          if (by_mask) binmask[bi] = 0ull;
          atomicAdd(&hcnt[bi], cnt);
        }
      }
    }
  }
  // Race draws of this wave's own candidates (the first waves to end their streams); the helper
  // waves draw the rest after the exchange.
  uint32_t nz = 0;
  if (order < kOwnDraws) {
    for (uint32_t base = 0; base < nc_here; base += 2u * kWaveSize) {
      draw_job(base, nc_here);
      nz = base + 2u * kWaveSize < nc_here ? base + 2u * kWaveSize : nc_here;
    }
  }
  if (lane == 0) {
    fs.wave_cand[wid] = ncand;
    fs.noise_done[wid] = nz;
    fs.bin_hi[wid] = wxc > -__builtin_inff() ? bmax + 1u : 0u;
  }
  lds_barrier();

  // ---- 4. Wave 0: status and the joint threshold. Waves 1-15: capture offsets, race draws ------
  // No barrier follows: each wave waits on LDS flags for exactly what it needs next.
  const bool capture = slot >= 0;
  // Race draws: jobs of 128 candidates of one wave (two independent Philox chains per lane,
  // whose latencies overlap), claimed by the helper waves from an LDS counter. The wave that
  // completes the last job picks the token (wave 0 when there is no job).
  constexpr uint32_t kJob = 2 * kWaveSize;
  const uint32_t l16 = lane & (kWaves - 1);
  const uint32_t nw0 = fs.wave_cand[l16];
  const uint32_t nw = nw0 < (uint32_t)LY::kCandCap ? nw0 : (uint32_t)LY::kCandCap;
  const uint32_t first = fs.noise_done[l16];  // drawn already: a multiple of 128, or all
  const uint32_t njobs = (nw - first + kJob - 1) / kJob;
  const uint32_t incl = wave_incl_scan(lane < (uint32_t)kWaves ? njobs : 0u, SumU32(), 0u);
  const uint32_t jobs = read_lane(incl, kWaves - 1);
  bool picker = false;
  if (wid == 0) {
    __builtin_amdgcn_s_setprio(3);
    const uint32_t w = lane & (kWaves - 1);
    const float m = row16_reduce(fs.wave_m[w], MaximumF32());
    const uint32_t ntot = row16_reduce(fs.wave_cand[w], SumU32());
    const bool over = __ballot(fs.wave_stash[w] > (uint32_t)kSpillPerWave ||
                               fs.wave_cand[w] > (uint32_t)LY::kCandCap) != 0;
    // A NaN logit: in the running maximum when top_p = 1, in the mass when top_p < 1.
    double zr = 0.0;
    if constexpr (NEED_P) zr = row16_reduce(fs.wave_z[w], SumF64());
    int32_t decision = kProceed;
    // With top_p < 1 the maximum comes from the candidates: trusted when it is +inf (a candidate
    // exists), but only without overflow otherwise.
    if (!(m == m) || m == __builtin_inff() || !(zr == zr)) {
      decision = kNonfinite;
    } else if (NEED_P && over) {
      decision = kFallback;
    } else if (m == -__builtin_inff()) {
      decision = kNoSupport;
    } else {
      const uint32_t kmax = key_of<E>(__float_as_uint(m) >> 16);
      double Z = 0.0;
      if constexpr (NEED_P) {
        // Z relative to the maximum: exp2(x c - m c) = exp2(x c - R c) * exp2(R c - m c), with
        // the rounded R c of the stream, so that its rounding cancels.
        Z = zr * exp2_fast(-(double)nrc - (double)m * (double)c);
        if (!(zr <= 1.0e300)) decision = kFallback;  // a float32 lane sum overflowed
      }
      if (over || kmax < theta_key || kmax - theta_key >= (uint32_t)kDBins) decision = kFallback;
      if (decision == kProceed) {
        const uint32_t dspan = kmax - theta_key;
        // With min-p, the bins past its cut cannot qualify: the scan stops at the last bin that
        // passes (every token below theta then fails min-p too, which the test below finds).
        const uint32_t dlim = mp > 0.0f ? min_p_last_bin(kmax, dspan, m, T, mp) : dspan;
        if (dlim < 4u * kWaveSize)
          bin_scan_wave0<NEED_P, 4, LY>(kmax, dspan, dlim, m, T, c, k, p, mp, Z, capture, hcnt, lds, fs);
        else
          bin_scan_wave0_wide<NEED_P, LY>(kmax, dspan, dlim, m, T, c, k, p, mp, Z, capture, hcnt, lds, fs);
        // Every token at or above theta is a candidate, so the scan is exact for the tie groups
        // it covers; the support is decided iff it also ends there: theta lies at or below the
        // k-th largest value (at least k candidates), or some candidate group below the support's
        // last group is excluded by top-p, min-p or top-k (with monotone predicates, every
        // token below theta is excluded too), or the value just below theta fails the scan's
        // min-p test (then so does every token below theta). Otherwise the general path decides
        // the row.
        bool below_fails_min_p = false;
        if (mp > 0.0f && theta_key > 0u) {
          const double tln_mp = (double)T * ln_fast((double)mp);
          const float xb = E::to_float(bits_of_key<E>(theta_key - 1u));
          below_fails_min_p = !(((double)xb - (double)m) >= tln_mp);
        }
        if (ntot < (uint32_t)k && !(fs.dstar < fs.dlow) && !below_fails_min_p) decision = kFallback;
        // No qualifying bin (bin 0 always qualifies in exact arithmetic; only a non-finite mass
        // could do this): the general path takes the row, and no loop below runs to d* = -1.
        if (fs.dstar < 0) decision = kFallback;
        if (decision == kProceed && BITS && capture && fs.L > (uint32_t)a.W) {
          // A support wider than W is also written as a bitmask: cleared here, and its bits set
          // by the capture. Waiting for every memory counter to drain means the clearing stores
          // have reached this CU's L2, where the capture's ORs and stores land, before any wave
          // can see scan_ready. (A device-scope release here wrote back the whole L2: 3 us more
          // on the B=256, V=151936 rows captured at W=512.)
          uint4* z = reinterpret_cast<uint4*>(a.bits + slot * a.bits_ld);
          const uint32_t n16 = (uint32_t)(bitmask_words(a.V) / 4);
          for (uint32_t i = lane; i < n16; i += kWaveSize) z[i] = make_uint4(0u, 0u, 0u, 0u);
          __builtin_amdgcn_s_waitcnt(0);
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        }
      }
    }
    if (decision != kProceed && lane == 0) fs.decision = decision;
    lds_publish(&fs.scan_ready, 1u);
    // Wave 0 picks the token once every race draw is done; it waits for them just before the
    // pick, after the row scalars below are read, so that none of that sits after the last draw.
    picker = true;
  } else {
    __builtin_amdgcn_s_setprio(2);
    if (capture && wid <= 4u) {
      // Exclusive prefix of every bin's count over the waves: wave w's first capture offset in
      // each tie group, relative to the group's base (waves 1-4; the other helpers start on the
      // race draws at once).
      uint16_t* cnt0 = reinterpret_cast<uint16_t*>(lds + LY::kOffTables);
      constexpr int kStride = LY::kTableStride / 2;  // u16 between two waves' tables
      uint32_t nbins = 0;  // bins any wave used
#pragma unroll
      for (int w = 0; w < kWaves; ++w) nbins = nbins > fs.bin_hi[w] ? nbins : fs.bin_hi[w];
      nbins = uniform_u32(nbins < (uint32_t)kDBins ? nbins : (uint32_t)kDBins);
      for (uint32_t j = tid - kWaveSize; j < nbins; j += 4u * kWaveSize) {
        uint32_t v[kWaves];
#pragma unroll
        for (int w = 0; w < kWaves; ++w) v[w] = cnt0[w * kStride + j];
        uint32_t acc = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          cnt0[w * kStride + j] = (uint16_t)acc;
          acc += v[w];
        }
      }
      lds_publish_step(&fs.prefix_done);
    }
    const uint32_t cwv = cw;
    const uint32_t* cand_all = reinterpret_cast<const uint32_t*>(lds + LY::kOffCand);
    for (;;) {
      const uint32_t q = lds_claim(&fs.job_next);
      if (q >= jobs) break;
      const uint32_t ww = (uint32_t)__popcll(__ballot(lane < (uint32_t)kWaves && incl <= q));
      const uint32_t c0 = read_lane(incl - njobs, (int)ww);
      const uint32_t nww = read_lane(nw, (int)ww);
      const uint32_t i0 = read_lane(first, (int)ww) + (q - c0) * kJob + lane;
      const uint32_t i1 = i0 + kWaveSize;
      const bool v0 = i0 < nww, v1 = i1 < nww;
      const uint32_t wd0 = v0 ? cand_all[ww * LY::kCandCap + i0] : 0u;
      const uint32_t wd1 = v1 ? cand_all[ww * LY::kCandCap + i1] : 0u;
      const uint32_t id0w = ww * cwv * 8u + (wd0 & 0x3FFFu);
      const uint32_t id1w = ww * cwv * 8u + (wd1 & 0x3FFFu);
      const uint32_t r0 = race_word(id0w, seed, pos);
      const uint32_t r1 = race_word(id1w, seed, pos);
      const uint32_t bi0 = key_of<E>(wd0 >> 16) - theta_key, bi1 = key_of<E>(wd1 >> 16) - theta_key;
      if (v0 && bi0 < (uint32_t)kDBins)
        atomicMax(reinterpret_cast<unsigned long long*>(&binbest[bi0]),
                  ((unsigned long long)(2u * (r0 >> 9) + 1u) << 32) | (unsigned long long)(~id0w));
      if (v1 && bi1 < (uint32_t)kDBins)
        atomicMax(reinterpret_cast<unsigned long long*>(&binbest[bi1]),
                  ((unsigned long long)(2u * (r1 >> 9) + 1u) << 32) | (unsigned long long)(~id1w));
      lds_publish_step(&fs.ready);
    }
  }
  const uint32_t wlim = a.wait_limit;
  // Wave 0 published scan_ready itself; every other wave waits for it (bounded).
  const bool scanned = lds_wait_at_least(&fs.scan_ready, 1u, wlim, &fs.aborted);
  if (scanned && fs.decision == kProceed) {
  const float m = waves_reduce(fs.wave_m, MaxOp());
  const uint32_t kmax = key_of<E>(__float_as_uint(m) >> 16);
  const uint32_t dspan = kmax - theta_key;
  const int32_t dstar = fs.dstar;
  const uint32_t L = fs.L;
  const double lnzs = fs.lnzs;
  const uint32_t* binbase = reinterpret_cast<const uint32_t*>(lds + LY::kOffBinBase);
  const double* bins = reinterpret_cast<const double*>(lds + LY::kOffBinS);
  const uint32_t W = (uint32_t)a.W;
  const float invT = 1.0f / T;

  // ---- 5. The pick, then the ordered capture of the opt-in row -----------------------------
  if (picker) {
    __builtin_amdgcn_s_setprio(3);
    if (lds_wait_at_least(&fs.ready, jobs * kStep, wlim, &fs.aborted)) {
    // The support is bins d = 0..d*; bin d holds key kmax - d at index dspan - d. Float32 scores
    // first; bins within kRaceMargin of the best are rescored in float64, ties -> lowest id.
    float b1 = -__builtin_inff(), b2 = -__builtin_inff();
    uint32_t p1 = 0u, d1 = 0u;  // best bin's ~id and d
    for (uint32_t d = lane; d <= (uint32_t)dstar; d += kWaveSize) {
      const uint64_t pk = binbest[dspan - d];
      if (pk == 0ull) continue;
      const float x = E::to_float(bits_of_key<E>(kmax - d));
      const float sc = (x - m) * invT + race_noise((float)(uint32_t)(pk >> 32) * 0x1p-24f);
      if (sc > b1) {
        b2 = b1;
        b1 = sc;
        p1 = (uint32_t)pk;
        d1 = d;
      } else if (sc > b2) {
        b2 = sc;
      }
    }
    const float t1 = wave_reduce(b1, [](float x, float y) { return x > y ? x : y; });
    const uint32_t src = (uint32_t)__builtin_ctzll(__ballot(b1 == t1));
    const float t2 = wave_reduce(lane == src ? b2 : b1, [](float x, float y) { return x > y ? x : y; });
    int32_t token = (int32_t)~read_lane(p1, (int)src);
    uint32_t td = read_lane(d1, (int)src);
    if (!(t1 - t2 > kRaceMargin)) {
      double bs = -__builtin_inf();
      int32_t bid = 0x7FFFFFFF;
      uint32_t bd = 0u;
      for (uint32_t d = lane; d <= (uint32_t)dstar; d += kWaveSize) {
        const uint64_t pk = binbest[dspan - d];
        if (pk == 0ull) continue;
        const float x = E::to_float(bits_of_key<E>(kmax - d));
        const float u32f = (float)(uint32_t)(pk >> 32) * 0x1p-24f;
        if ((x - m) * invT + race_noise(u32f) < t1 - kRaceMargin) continue;
        const double sv = ((double)x - (double)m) / (double)T;
        const double sc = sv - log(-log((double)(uint32_t)(pk >> 32) * 0x1p-24));
        const int32_t id = (int32_t)~(uint32_t)pk;
        if (sc > bs || (sc == bs && id < bid)) {
          bs = sc;
          bid = id;
          bd = d;
        }
      }
      const double wt = wave_reduce(bs, [](double x, double y) { return x > y ? x : y; });
      token = wave_reduce(bs == wt ? bid : 0x7FFFFFFF, [](int32_t x, int32_t y) { return x < y ? x : y; });
      td = wave_reduce(bs == wt && bid == token ? bd : 0u, MaxU32());
    }
    // Written at once (thread 0, the same thread that writes an ABORTED status over them after
    // the row's last barrier, in program order, should any wait of the row give up).
    if (lane == 0) {
      a.tokens[b] = token;
      a.row_status[b] = (capture && L > W) ? TSC_ROW_OVERFLOW : TSC_ROW_OK;
      if (capture) {
        a.lengths[slot] = (int32_t)(L < W ? L : W);
        a.selected_logprob[slot] = (float)(bins[dspan - td] - lnzs);
      }
    }
    }
  }
  if constexpr (COMPACT) {
  // Capture (compaction mode): every wave stages its own list from the ranks it took before the
  // exchange, then the waves copy the stage out in slices.
  __builtin_amdgcn_s_setprio(1);
  if (capture && lds_wait_at_least(&fs.prefix_done, 4u * kStep, wlim, &fs.aborted)) {
    // A candidate survives iff its key >= kmax - d* (bins failing min-p lie beyond d*), i.e. its
    // value >= x_cut (-0 and +0 compare equal, as their keys do).
    const float x_cut = E::to_float(bits_of_key<E>(kmax - (uint32_t)dstar));
    int32_t* out_ids = a.packed_ids + slot * a.W;
    float* out_lp = a.logprobs ? a.logprobs + slot * a.W : nullptr;
    uint32_t* stage = reinterpret_cast<uint32_t*>(lds + LY::kOffStage);
    uint32_t* const brow = (BITS && L > W) ? a.bits + slot * a.bits_ld : nullptr;
    if (BITS && brow != nullptr) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    {
      // Each wave places its own list: a survivor's position is its bin's base (tokens with
      // larger keys) + the bin's members in earlier segments (the wave's table, now the prefix
      // over the waves) + its rank in the wave. Its packed word (id | bi << 18) goes to the LDS
      // stage; once every list is staged, the stage is copied out with coalesced stores.
      const uint32_t* cand_w = reinterpret_cast<const uint32_t*>(lds + LY::kOffCand) + wid * LY::kCandCap;
      const uint16_t* pre_w = reinterpret_cast<const uint16_t*>(lds + LY::kOffTables + wid * LY::kTableStride);
#pragma unroll
      for (int cc = 0; cc < 2 * kRankRegs; ++cc) {
        if ((uint32_t)cc * kWaveSize < nc_here) {
          const uint32_t i = (uint32_t)cc * kWaveSize + lane;
          const uint32_t wd = i < nc_here ? cand_w[i] : 0xFF800000u;
          if (i < nc_here && __uint_as_float(wd & 0xFFFF0000u) >= x_cut) {
            const uint32_t bi = key_of<E>(wd >> 16) - theta_key;
            const uint32_t r = (crank[cc >> 1] >> ((cc & 1) * 16)) & 0xFFFFu;
            const uint32_t at = binbase[bi] + pre_w[bi] + r;
            const uint32_t id = id0 + (wd & 0x3FFFu);
            if (at < (uint32_t)LY::kStageCap) {
              stage[at] = id | (bi << 18);
            } else if (at < W) {
              out_ids[at] = (int32_t)id;
              if (out_lp) out_lp[at] = (float)(bins[bi] - lnzs);
            }
          }
        }
      }
      lds_publish_step(&fs.staged);
    }
    // Copy-out of the stage, in slices of 1024 positions.
    const uint32_t nl = L < W ? L : W;
    const uint32_t nout = nl < (uint32_t)LY::kStageCap ? nl : (uint32_t)LY::kStageCap;
    // Slices are claimed by the waves in turn. Four entries per lane at a time: their stage
    // words, then their bins' logprobs, are read together. A capture of at least kNtStoreMin
    // entries is written with nontemporal stores: these coalesced rows stream to memory as they
    // are written instead of staying dirty in L2 until the kernel's end, whose release then has
    // to write them back (B=256 rows of width 8192, 16.8 MB: 35.8 -> 33.8 us). Scattered stores
    // (stash mode) stay ordinary: nontemporal there cost the B=256, V=151936 batch 1 us. The two store kinds are separate instantiations
    // of the loop: a run-time choice between two otherwise equal stores is merged by the
    // compiler into one ordinary store.
    auto copy_out = [&](auto nt_tag) {
      constexpr bool kNt = decltype(nt_tag)::value;
      for (;;) {
        const uint32_t sl = lds_claim(&fs.copy_next);
        if (sl * 1024u >= nout) break;
        const uint32_t end = (sl + 1u) * 1024u < nout ? (sl + 1u) * 1024u : nout;
        for (uint32_t j0 = sl * 1024u + lane; j0 < end; j0 += 4u * kWaveSize) {
          uint32_t e[4];
          double bl[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t j = j0 + (uint32_t)t * kWaveSize;
            e[t] = j < end ? stage[j] : 0u;
          }
#pragma unroll
          for (int t = 0; t < 4; ++t) bl[t] = out_lp ? bins[e[t] >> 18] : 0.0;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const uint32_t j = j0 + (uint32_t)t * kWaveSize;
            if (j < end) {
              if constexpr (kNt) {
                __builtin_nontemporal_store((int32_t)(e[t] & 0x3FFFFu), &out_ids[j]);
                if (out_lp) __builtin_nontemporal_store((float)(bl[t] - lnzs), &out_lp[j]);
              } else {
                out_ids[j] = (int32_t)(e[t] & 0x3FFFFu);
                if (out_lp) out_lp[j] = (float)(bl[t] - lnzs);
              }
            }
          }
        }
      }
    };
    if (nout > 0u && lds_wait_at_least(&fs.staged, (uint32_t)kWaves * kStep, wlim, &fs.aborted)) {
      if (nl >= kNtStoreMin)
        copy_out(BoolTag<true>{});
      else
        copy_out(BoolTag<false>{});
    }
    // Bitmask bits, one candidate list per claim, by the waves with no stage slice left: off
    // the path from the ranking to the copy-out.
    if (BITS && brow != nullptr) {
      for (;;) {
        const uint32_t cj = lds_claim(&fs.bits_next);
        if (cj >= (uint32_t)kWaves) break;
        const uint32_t ncj0 = fs.wave_cand[cj];
        const uint32_t ncj = ncj0 < (uint32_t)LY::kCandCap ? ncj0 : (uint32_t)LY::kCandCap;
        support_bits_of_list(reinterpret_cast<const uint32_t*>(lds + LY::kOffCand) + cj * LY::kCandCap,
                                   ncj, x_cut, cj * cw * 8u, brow);
      }
    }
  }
  } else {
  // Capture (stash mode): one job per wave's candidate list, claimed by whichever waves are free.
  // A survivor's position is its bin's base (tokens with larger keys) + the bin's members in
  // earlier segments (smaller ids: the prefix over the waves) + its rank in its wave.
  __builtin_amdgcn_s_setprio(1);
  if (capture && lds_wait_at_least(&fs.prefix_done, 4u * kStep, wlim, &fs.aborted)) {
    // A candidate survives iff its key >= kmax - d* (bins failing min-p lie beyond d*), i.e. its
    // value >= x_cut (-0 and +0 compare equal, as their keys do).
    const float x_cut = E::to_float(bits_of_key<E>(kmax - (uint32_t)dstar));
    int32_t* out_ids = a.packed_ids + slot * a.W;
    float* out_lp = a.logprobs ? a.logprobs + slot * a.W : nullptr;
    uint32_t* const brow = (BITS && L > W) ? a.bits + slot * a.bits_ld : nullptr;
    if (BITS && brow != nullptr) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    for (;;) {
      const uint32_t cj = lds_claim(&fs.cap_next);
      if (cj >= (uint32_t)kWaves) break;
      const uint32_t ncj0 = fs.wave_cand[cj];
      const uint32_t ncj = ncj0 < (uint32_t)LY::kCandCap ? ncj0 : (uint32_t)LY::kCandCap;
      const uint32_t* cand_c = reinterpret_cast<const uint32_t*>(lds + LY::kOffCand) + cj * LY::kCandCap;
      const uint16_t* bincnt_c =
          reinterpret_cast<const uint16_t*>(lds + LY::kOffTables + cj * LY::kTableStride);
      const uint16_t* rank_c =
          reinterpret_cast<const uint16_t*>(lds + LayoutStash::kOffRank) + cj * LY::kCandCap;
      const uint32_t id0c = cj * cw * 8u;
      for (uint32_t i = lane; i < ncj; i += kWaveSize) {
        const uint32_t wd = cand_c[i];
        const float x = __uint_as_float(wd & 0xFFFF0000u);
        if (!(x >= x_cut)) continue;
        const uint32_t bi = key_of<E>(wd >> 16) - theta_key;
        const uint32_t at = binbase[bi] + bincnt_c[bi] + rank_c[i];
        if (at < W) {
          out_ids[at] = (int32_t)(id0c + (wd & 0x3FFFu));
          if (out_lp) out_lp[at] = (float)(bins[bi] - lnzs);
        }
      }
      if (BITS && brow != nullptr) support_bits_of_list(cand_c, ncj, x_cut, id0c, brow);
    }
  }
  }
  }
  // Every wave arrives here exactly once, whatever its waits gave: the row's outputs are decided
  // after this barrier, by what the workgroup as a whole saw.
  lds_barrier();
  if (fs.aborted != 0u) {
    finish_empty_row(a, b, slot, TSC_ROW_ABORTED);
    return true;
  }
  const int32_t decision = fs.decision;
  if (decision == kNonfinite || decision == kNoSupport) {
    finish_empty_row(a, b, slot, decision == kNonfinite ? TSC_ROW_NONFINITE : TSC_ROW_NO_SUPPORT);
    return true;
  }
  return decision == kProceed;
}


// k: the row's top_k, INT32_MAX when the filter is off; kv: the top_k the cutoff theta is chosen
// for (k itself up to the compaction range, else kOffK in stash mode).
template <int LOADS, bool BITS>
__device__ __forceinline__ bool fast_row_dispatch(const SampleArgs& a, int64_t b, int64_t& slot,
                                                  float T, int32_t k, int32_t kv, float p, float mp,
                                                  uint64_t seed, uint64_t pos, unsigned char* lds,
                                                  FastShared& fs) {
  if (kv <= kFastMaxK)
    return p < 1.0f ? fast_row_bf16<true, false, LOADS, BITS>(a, b, slot, T, k, kv, p, mp, seed, pos, lds, fs)
                    : fast_row_bf16<false, false, LOADS, BITS>(a, b, slot, T, k, kv, p, mp, seed, pos, lds, fs);
  return p < 1.0f ? fast_row_bf16<true, true, LOADS, BITS>(a, b, slot, T, k, kv, p, mp, seed, pos, lds, fs)
                  : fast_row_bf16<false, true, LOADS, BITS>(a, b, slot, T, k, kv, p, mp, seed, pos, lds, fs);
}

}  // namespace tsc

#include "tsc_fast_f32.h"
#include "tsc_greedy.h"

namespace tsc {

// BITS: the call passed a support bitmask buffer (a separate instantiation, so that calls without
// one run no bitmask code at all).
template <int DT, bool BITS>
__global__ void __launch_bounds__(kThreads) sample_fast_kernel(SampleArgs a) {
  // The dynamic buffer starts after the static LDS; 256-byte alignment keeps every 16-byte
  // stash access aligned (and the bank mapping of the layout fixed) whatever FastShared's size.
  extern __shared__ __attribute__((aligned(256))) uint64_t dyn[];
  __shared__ FastShared fs;
  unsigned char* lds = reinterpret_cast<unsigned char*>(dyn);
  const int64_t b = blockIdx.x;
  int64_t slot = -2;  // looked up inside the fast path, after its loads are issued
  if constexpr (DT == TSC_DTYPE_BF16) {
    const float T = a.temperature[b];
    const int32_t k = a.top_k[b];
    const float p = a.top_p[b];
    const float mp = a.min_p[b];
    const uint64_t seed = a.seeds[b], pos = a.positions[b];
    if (greedy_eligible<DT>(a, T, p, mp)) {
      slot = find_capture_slot(a, b, fs.red);
      greedy_row<DT>(a, b, slot, fs.red);
      return;
    }
    // top_k off (<= 0 or >= V) or beyond the compaction range: the cutoff is chosen as for
    // top_k = kOffK, and the row is served here when top-p or min-p ends its support among
    // the candidates (checked after the scan; otherwise the general path takes it). A row with
    // no filter at all (support = every finite token) goes to the general path directly.
    const bool k_on = k >= 1 && (int64_t)k < a.V;
    const int32_t keff = k_on ? k : 0x7FFFFFFF;
    const int32_t kv = (k_on && k <= kCompactMaxK) ? k : kOffK;
    const bool eligible = row_params_valid(T, p, mp) && T > 0.0f &&
                          ((k_on && k <= kCompactMaxK) || p < 1.0f || mp > 0.0f) &&
                          a.V >= kFastMinV && a.V <= kFastMaxV &&
                          (a.V & 7) == 0 && (a.ld & 7) == 0 &&
                          (reinterpret_cast<uintptr_t>(a.logits) & 15u) == 0;
    if (eligible) {
      const bool done =
          a.V <= kShortMaxV
              ? fast_row_dispatch<kShortLoads, BITS>(a, b, slot, T, keff, kv, p, mp, seed, pos, lds, fs)
              : fast_row_dispatch<kFastLoads, BITS>(a, b, slot, T, keff, kv, p, mp, seed, pos, lds, fs);
      if (done) return;
      __syncthreads();  // the general path reuses the LDS
    }
  } else {
    const float T = a.temperature[b];
    const int32_t k = a.top_k[b];
    const float p = a.top_p[b];
    const float mp = a.min_p[b];
    const uint64_t seed = a.seeds[b], pos = a.positions[b];
    if (greedy_eligible<DT>(a, T, p, mp)) {
      slot = find_capture_slot(a, b, fs.red);
      greedy_row<DT>(a, b, slot, fs.red);
      return;
    }
    // As for bfloat16 rows: top_k off or above kF32MaxK chooses the cutoff as for kF32OffK.
    const bool k_on = k >= 1 && (int64_t)k < a.V;
    const int32_t keff = k_on ? k : 0x7FFFFFFF;
    const int32_t kv = (k_on && k <= kF32MaxK) ? k : kF32OffK;
    const bool eligible = row_params_valid(T, p, mp) && T > 0.0f &&
                          ((k_on && k <= kF32MaxK) || p < 1.0f || mp > 0.0f) &&
                          a.V >= kF32MinV && a.V <= kF32MaxV && (a.V & 3) == 0 &&
                          (a.ld & 3) == 0 && (reinterpret_cast<uintptr_t>(a.logits) & 15u) == 0;
    if (eligible) {
      bool done;
      if (a.V <= kF32ShortMaxV)
        done = p < 1.0f
                   ? fast_row_f32<true, kF32ShortLoads, BITS>(a, b, slot, T, keff, kv, p, mp, seed, pos, lds, fs)
                   : fast_row_f32<false, kF32ShortLoads, BITS>(a, b, slot, T, keff, kv, p, mp, seed, pos, lds, fs);
      else
        done = p < 1.0f
                   ? fast_row_f32<true, kF32LongLoads, BITS>(a, b, slot, T, keff, kv, p, mp, seed, pos, lds, fs)
                   : fast_row_f32<false, kF32LongLoads, BITS>(a, b, slot, T, keff, kv, p, mp, seed, pos, lds, fs);
      if (done) return;
      __syncthreads();  // the general path reuses the LDS
    }
  }
  if (slot == -2) slot = find_capture_slot(a, b, fs.red);
  GeneralShared* sh = reinterpret_cast<GeneralShared*>(lds + kGeneralDynLds);
  general_row<DT, BITS>(a, b, slot, dyn, *sh);
}

}  // namespace tsc
