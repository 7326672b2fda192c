// Device helpers shared by the sampler kernels: orderable keys, the Philox4x32-10 generator and
// block-wide reductions for 1024-thread workgroups of 64-wide wavefronts (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tsc.h"

namespace tsc {

constexpr int kThreads = 1024;
constexpr int kWaveSize = 64;
constexpr int kWaves = kThreads / kWaveSize;
// Captures (a row's packed ids and logprobs, or a slot of the support CSR) of at least this many
// entries, written as coalesced rows, use nontemporal stores.
constexpr uint32_t kNtStoreMin = 4096;

// A compile-time flag passed to a generic lambda, which then instantiates one body per value.
template <bool B>
struct BoolTag {
  static constexpr bool value = B;
};

// ---- Logit element types -------------------------------------------------------------------
// A key is an unsigned integer image of a logit whose order is the order of the values, with -0
// and +0 mapped to one key (ties are judged on the value, so the two zeros tie).
template <int DT>
struct Elem;

template <>
struct Elem<TSC_DTYPE_BF16> {
  using Bits = uint16_t;
  static constexpr int kVec = 8;  // elements per 16-byte load
  static constexpr int kKeyBits = 16;
  static constexpr uint32_t kSign = 0x8000u, kMask = 0xFFFFu, kExpMask = 0x7F80u;
  static constexpr uint32_t kNegInf = 0xFF80u;
  __device__ static inline float to_float(uint32_t b) { return __uint_as_float(b << 16); }
};

template <>
struct Elem<TSC_DTYPE_F32> {
  using Bits = uint32_t;
  static constexpr int kVec = 4;
  static constexpr int kKeyBits = 32;
  static constexpr uint32_t kSign = 0x80000000u, kMask = 0xFFFFFFFFu, kExpMask = 0x7F800000u;
  static constexpr uint32_t kNegInf = 0xFF800000u;
  __device__ static inline float to_float(uint32_t b) { return __uint_as_float(b); }
};

template <class E>
__device__ inline uint32_t key_of(uint32_t b) {
  if (b == E::kSign) b = 0;  // -0 -> +0
  return (b & E::kSign) ? (~b & E::kMask) : (b | E::kSign);
}

template <class E>
__device__ inline uint32_t bits_of_key(uint32_t k) {
  return (k & E::kSign) ? (k ^ E::kSign) : (~k & E::kMask);
}

template <class E>
__device__ inline bool is_finite_bits(uint32_t b) {
  return (b & E::kExpMask) != E::kExpMask;
}

// ---- Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11, section 4) ---------------------------
// Per round, with (hi_a, lo_a) = M0 * X0 and (hi_b, lo_b) = M1 * X2 as 64-bit products:
// X' = (hi_b ^ X1 ^ K0, lo_b, hi_a ^ X3 ^ K1, lo_a); the key advances by the Weyl constants.
__device__ inline uint4 philox4x32_10(uint4 x, uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    // One full 32x32 -> 64-bit product per multiplier (v_mad_u64_u32) gives both halves.
    const uint64_t pa = (uint64_t)M0 * x.x, pb = (uint64_t)M1 * x.z;
    x = make_uint4((uint32_t)(pb >> 32) ^ x.y ^ k0, (uint32_t)pb, (uint32_t)(pa >> 32) ^ x.w ^ k1,
                   (uint32_t)pa);
  }
  return x;
}

// The race uniform of token `id` in a row: Philox keyed by the seed, counter (id / 4, 0,
// position), output word id % 4; the 23 high bits k give u = (2k + 1) / 2^24 in (0, 1).
__device__ inline uint32_t race_word(uint32_t id, uint64_t seed, uint64_t position) {
  const uint4 r = philox4x32_10(
      make_uint4(id >> 2, 0u, (uint32_t)position, (uint32_t)(position >> 32)),
      (uint32_t)seed, (uint32_t)(seed >> 32));
  const uint32_t j = id & 3u;
  return j == 0 ? r.x : j == 1 ? r.y : j == 2 ? r.z : r.w;
}

__device__ inline double race_uniform(uint32_t id, uint64_t seed, uint64_t position) {
  return (double)(2u * (race_word(id, seed, position) >> 9) + 1u) * 0x1p-24;
}

// Workgroup barrier that orders LDS only: global loads still in flight stay in flight. Every
// block-level exchange in these kernels goes through LDS, so this is the barrier they use.
__device__ inline void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ---- Wavefront primitives on DPP (gfx9 encodings; every lane of the wave must be active) -----
// A DPP move reads another lane's register in the same VALU instruction, without the LDS round
// trip of a ds_bpermute shuffle. `old` is what lanes without a valid source keep.
namespace dpp {
constexpr int kQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowRor4 = 0x124, kRowRor8 = 0x128;
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowShl4 = 0x104;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;
}  // namespace dpp

template <int CTRL, int ROW_MASK = 0xF, class T>
__device__ inline T dpp_mov(T old, T src) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 8, "32- or 64-bit values");
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, old),
                                                             __builtin_bit_cast(int, src), CTRL,
                                                             ROW_MASK, 0xF, false));
  } else {
    const uint64_t o = __builtin_bit_cast(uint64_t, old), v = __builtin_bit_cast(uint64_t, src);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)o, (int)(uint32_t)v,
                                                              CTRL, ROW_MASK, 0xF, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(o >> 32),
                                                              (int)(uint32_t)(v >> 32), CTRL,
                                                              ROW_MASK, 0xF, false);
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  }
}

// The value held by lane (lane ^ J), J = 1, 2, ..., 32, in VALU instructions only: DPP within a
// row of 16 lanes (xor 4 takes the row shift in each direction and keeps the one in range), and
// gfx950's permlane swaps across rows (xor 16: odd rows of one copy with even rows of the other;
// xor 32: the two halves of the wave).
template <int J>
__device__ inline uint32_t xor_lanes(uint32_t x) {
  static_assert(J == 1 || J == 2 || J == 4 || J == 8 || J == 16 || J == 32, "lane xor");
  const uint32_t lane = threadIdx.x & 63u;
  if constexpr (J == 1) {
    return dpp_mov<dpp::kQuadSwap1>(x, x);
  } else if constexpr (J == 2) {
    return dpp_mov<dpp::kQuadSwap2>(x, x);
  } else if constexpr (J == 4) {
    const uint32_t up = dpp_mov<dpp::kRowShl4>(x, x), dn = dpp_mov<dpp::kRowShr4>(x, x);
    return (lane & 4u) ? dn : up;
  } else if constexpr (J == 8) {
    return dpp_mov<dpp::kRowRor8>(x, x);
  } else if constexpr (J == 16) {
    const auto sw = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return (lane & 16u) ? sw[0] : sw[1];
  } else {
    const auto sw = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (lane & 32u) ? sw[0] : sw[1];
  }
}

template <int J>
__device__ inline uint64_t xor_lanes(uint64_t x) {
  return ((uint64_t)xor_lanes<J>((uint32_t)(x >> 32)) << 32) | xor_lanes<J>((uint32_t)x);
}

template <class T>
__device__ inline T read_lane(T v, int lane) {
  if constexpr (sizeof(T) == 4) {
    return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
  } else {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), lane);
    return __builtin_bit_cast(T, ((uint64_t)hi << 32) | lo);
  }
}

// op over the 64 lanes; every lane receives the result. op must be commutative and associative
// (the combination order is fixed, so a floating-point sum is reproducible).
template <class T, class Op>
__device__ inline T wave_reduce(T v, Op op) {
  v = op(v, dpp_mov<dpp::kQuadSwap1>(v, v));
  v = op(v, dpp_mov<dpp::kQuadSwap2>(v, v));
  v = op(v, dpp_mov<dpp::kRowRor4>(v, v));
  v = op(v, dpp_mov<dpp::kRowRor8>(v, v));
  return op(op(read_lane(v, 0), read_lane(v, 16)), op(read_lane(v, 32), read_lane(v, 48)));
}

// Inclusive scan under op with identity `id` (lane i receives op over lanes 0..i).
template <class T, class Op>
__device__ inline T wave_incl_scan(T v, Op op, T id) {
  v = op(v, dpp_mov<dpp::kRowShr1>(id, v));
  v = op(v, dpp_mov<dpp::kRowShr2>(id, v));
  v = op(v, dpp_mov<dpp::kRowShr4>(id, v));
  v = op(v, dpp_mov<dpp::kRowShr8>(id, v));
  v = op(v, dpp_mov<dpp::kRowBcast15, 0xA>(id, v));
  v = op(v, dpp_mov<dpp::kRowBcast31, 0xC>(id, v));
  return v;
}

// ---- Per-wave partials in LDS ------------------------------------------------------------------
// A 64-lane read of one LDS word (a broadcast) occupies the LDS as long as a read of 64 distinct
// words, so 16 waves each reading 16 partials one by one keep it busy for ~500 clocks per 32-bit
// array. Instead every wave reads the 16 partials once (lane i holds s[i % 16]: four copies of
// the row of 16 lanes) and combines them on DPP within a row.
static_assert(kWaves == 16, "the partials of a workgroup fill one DPP row of 16 lanes");

// Reduction over the first 16 lanes, for data that every row of 16 lanes holds alike (lane l
// holding entry l % 16): four DPP steps inside each row (a fixed order), then lane 0.
template <class T, class Op>
__device__ inline T row16_reduce(T v, Op op) {
  v = op(v, dpp_mov<dpp::kQuadSwap1>(v, v));
  v = op(v, dpp_mov<dpp::kQuadSwap2>(v, v));
  v = op(v, dpp_mov<dpp::kRowRor4>(v, v));
  v = op(v, dpp_mov<dpp::kRowRor8>(v, v));
  return read_lane(v, 0);
}

// op over s[0..15]; the same value (wave-uniform, identical in every wave) for every lane.
template <class T, class Op>
__device__ inline T waves_reduce(const T* s, Op op) {
  return row16_reduce(s[threadIdx.x & (kWaves - 1)], op);
}

// op over s[0..w-1] for the calling wave w (`id` for wave 0); `total` receives op over all 16.
template <class T, class Op>
__device__ inline T waves_prefix(const T* s, Op op, T id, T& total) {
  T v = s[threadIdx.x & (kWaves - 1)];
  v = op(v, dpp_mov<dpp::kRowShr1>(id, v));
  v = op(v, dpp_mov<dpp::kRowShr2>(id, v));
  v = op(v, dpp_mov<dpp::kRowShr4>(id, v));
  v = op(v, dpp_mov<dpp::kRowShr8>(id, v));
  total = read_lane(v, kWaves - 1);
  const int w = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWaveSize));
  return w == 0 ? id : read_lane(v, w - 1);
}

// ---- Block reductions (fixed order, hence deterministic) -----------------------------------
// Reduces `v` over the workgroup; every thread receives the result. `scratch` is shared memory
// of at least kWaves * 8 bytes; the leading barrier makes back-to-back calls safe.
template <class T, class Op>
__device__ inline T block_reduce(T v, Op op, uint64_t* scratch) {
  v = wave_reduce(v, op);
  T* s = reinterpret_cast<T*>(scratch);
  lds_barrier();
  if ((threadIdx.x & (kWaveSize - 1)) == 0) s[threadIdx.x / kWaveSize] = v;
  lds_barrier();
  return waves_reduce(s, op);
}

struct MaxOp {
  template <class T>
  __device__ T operator()(T a, T b) const { return a > b ? a : b; }
};
struct MinOp {
  template <class T>
  __device__ T operator()(T a, T b) const { return a < b ? a : b; }
};
struct SumOp {
  template <class T>
  __device__ T operator()(T a, T b) const { return a + b; }
};

}  // namespace tsc
