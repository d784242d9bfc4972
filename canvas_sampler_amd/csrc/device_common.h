// Device-side building blocks of the canvas sampler (gfx950, wave64):
// Philox4x32-10, the uniform/Gumbel maps of the random protocol, and wave64
// reductions. Written for this library; shares nothing with the oracle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

constexpr int kWave = 64;

// Vocabulary geometry of the sampling protocol. A stripe is 512 consecutive
// ids = 64 slots of 8 ids; one wave64 reads one stripe with one 16-byte load
// per lane (bf16), so every load is fully coalesced. A chunk is 8 consecutive
// stripes (4096 ids); block j = 64 * chunk + slot gathers one slot across the
// 8 stripes of its chunk (64 ids), so a lane of a wave streaming a chunk holds
// exactly one whole block in its registers. For an id v that is
// j = 64 * (v >> 12) + ((v >> 3) & 63).
constexpr int kSlotIds = 8;
constexpr int kSlots = 64;
constexpr int kStripeIds = kSlotIds * kSlots;        // 512
constexpr int kChunkStripes = 8;
constexpr int kChunkIds = kStripeIds * kChunkStripes;  // 4096

// Counter word 3 of each random draw.
constexpr uint32_t kTagInit = 0;
constexpr uint32_t kTagBlock = 1;
constexpr uint32_t kTagElem = 2;
constexpr uint32_t kTagRenoise = 3;
constexpr uint32_t kTagCanvas = 4;   // seed of a later canvas of a block-autoregressive stream

struct Words4 {
  uint32_t w[4];
};

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two 32x32
// multiplies whose halves are mixed with the other counter words and the
// round key; the key advances by the Weyl constants between rounds. The key is
// uniform across a wave in every use here, so its additions stay scalar.
__device__ __forceinline__ Words4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c0;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c2;
    const uint32_t n0 = static_cast<uint32_t>(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = static_cast<uint32_t>(p0 >> 32) ^ c3 ^ k1;
    c1 = static_cast<uint32_t>(p1);
    c3 = static_cast<uint32_t>(p0);
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  Words4 out;
  out.w[0] = c0;
  out.w[1] = c1;
  out.w[2] = c2;
  out.w[3] = c3;
  return out;
}

// U = (2*(w >> 9) + 1) * 2^-24, strictly inside (0,1) and exact in fp32.
__device__ __forceinline__ float uniform_open01(uint32_t w) {
  return static_cast<float>(((w >> 9) << 1) | 1u) * 5.9604644775390625e-8f;
}

// Standard Gumbel -ln(-ln U) with the hardware log2 (v_log_f32). Large
// variates come from U close to 1, where -ln U is tiny and must keep its
// relative accuracy; v_log_f32 does (checked over all 2^23 values of U against
// fp64: error at most 2.9e-7 * max(1, |G|), the same as with library log1p).
__device__ __forceinline__ float gumbel(uint32_t w) {
  constexpr float kLn2f = 0.69314718055994530942f;
  const float u = uniform_open01(w);
  const float e = -kLn2f * __builtin_amdgcn_logf(u);  // -ln U > 0
  return -kLn2f * __builtin_amdgcn_logf(e);
}

// floor(w * V / 2^32): a uniform vocabulary id.
__device__ __forceinline__ int32_t uniform_token(uint32_t w, uint32_t vocab) {
  return static_cast<int32_t>(__umulhi(w, vocab));
}

// max(a, b, c) as one v_max3_f32. Written as inline asm because the compiler
// otherwise canonicalizes every operand that came from integer bit operations
// or a raw load (one extra v_max per value) to honour IEEE signalling-NaN
// rules; logits are never NaN, so the plain instruction is exact here.
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// max(a, b) as one v_max_f32, for values that are never NaN (see max3_raw).
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// ---- cross-lane moves and wave64 reductions ----
// All moves stay in the VALU: DPP within rows of 16 lanes, and gfx950's
// v_permlane16_swap / v_permlane32_swap across rows and halves. Neither goes
// through the LDS crossbar, whose round trip (ds_bpermute) would dominate the
// short reductions that end a pass.

// DPP move of v with control CTRL over all rows and banks; lanes whose source
// lies outside their row keep v.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

constexpr int kDppXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppShl4 = 0x104;   // row_shl:4, lane i <- lane i+4 of its row
constexpr int kDppShr4 = 0x114;   // row_shr:4, lane i <- lane i-4 of its row
constexpr int kDppRor4 = 0x124;   // row_ror:4, lane i <- lane (i-4) mod 16 of its row
constexpr int kDppXor8 = 0x128;   // row_ror:8, lane i <- lane i^8

// The value of lane (lane ^ J), J a power of two below 64.
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (J == 1) {
    return dpp_mov<kDppXor1>(v);
  } else if constexpr (J == 2) {
    return dpp_mov<kDppXor2>(v);
  } else if constexpr (J == 4) {
    const uint32_t up = dpp_mov<kDppShl4>(v), down = dpp_mov<kDppShr4>(v);
    return (__lane_id() & 4) ? down : up;
  } else if constexpr (J == 8) {
    return dpp_mov<kDppXor8>(v);
  } else if constexpr (J == 16) {
    // [0] holds rows (0,0,2,2) of v, [1] rows (1,1,3,3)
    const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (__lane_id() & 16) ? p[0] : p[1];
  } else {
    static_assert(J == 32, "lane_xor: J must be a power of two below 64");
    // [0] holds the low half of v in both halves, [1] the high half
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (__lane_id() & 32) ? p[0] : p[1];
  }
}

template <int J>
__device__ __forceinline__ uint64_t lane_xor64(uint64_t v) {
  const uint32_t lo = lane_xor<J>(static_cast<uint32_t>(v));
  const uint32_t hi = lane_xor<J>(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ float f32_of(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t u32_of(float f) { return __float_as_uint(f); }

// Maximum over the wave of values that are never NaN.
__device__ __forceinline__ float wave_max(float v) {
#define DG_STEP(C) v = max_raw(v, f32_of(dpp_mov<C>(u32_of(v))))
  DG_STEP(kDppXor8); DG_STEP(kDppRor4); DG_STEP(kDppXor2); DG_STEP(kDppXor1);
#undef DG_STEP
  const auto p = __builtin_amdgcn_permlane16_swap(u32_of(v), u32_of(v), false, false);
  v = max_raw(f32_of(p[0]), f32_of(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(u32_of(v), u32_of(v), false, false);
  return max_raw(f32_of(q[0]), f32_of(q[1]));
}

__device__ __forceinline__ int wave_min_int(int v) {
#define DG_STEP(C) v = min(v, static_cast<int>(dpp_mov<C>(static_cast<uint32_t>(v))))
  DG_STEP(kDppXor8); DG_STEP(kDppRor4); DG_STEP(kDppXor2); DG_STEP(kDppXor1);
#undef DG_STEP
  const auto p = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(v), static_cast<uint32_t>(v), false, false);
  v = min(static_cast<int>(p[0]), static_cast<int>(p[1]));
  const auto q = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(v), static_cast<uint32_t>(v), false, false);
  return min(static_cast<int>(q[0]), static_cast<int>(q[1]));
}

template <int C>
__device__ __forceinline__ double dpp_mov_f64(double v) {
  const uint64_t b = __double_as_longlong(v);
  const uint32_t lo = dpp_mov<C>(static_cast<uint32_t>(b));
  const uint32_t hi = dpp_mov<C>(static_cast<uint32_t>(b >> 32));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

// Sum over the wave; every lane returns the same bits.
__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_mov_f64<kDppXor8>(v);
  v += dpp_mov_f64<kDppRor4>(v);
  v += dpp_mov_f64<kDppXor2>(v);
  v += dpp_mov_f64<kDppXor1>(v);
  uint64_t b = __double_as_longlong(v);
  const auto plo = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(b), static_cast<uint32_t>(b), false, false);
  const auto phi = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(b >> 32), static_cast<uint32_t>(b >> 32),
                                                    false, false);
  v = __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(phi[0]) << 32) | plo[0])) +
      __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(phi[1]) << 32) | plo[1]));
  b = __double_as_longlong(v);
  const auto qlo = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(b), static_cast<uint32_t>(b), false, false);
  const auto qhi = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(b >> 32), static_cast<uint32_t>(b >> 32),
                                                    false, false);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(qhi[0]) << 32) | qlo[0])) +
         __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(qhi[1]) << 32) | qlo[1]));
}

// (score, index) arg-max as one unsigned 64-bit key: the score's bits made
// order-preserving (both zeros as +0, so equal scores tie) above the
// complemented index, so that the larger key has the higher score and, among
// equal scores, the lower index. Indices are non-negative.
__device__ __forceinline__ uint64_t argmax_key(float score, int idx) {
  const uint32_t b = score == 0.0f ? 0u : __float_as_uint(score);
  const uint32_t ord = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return (static_cast<uint64_t>(ord) << 32) | static_cast<uint32_t>(~idx);
}

__device__ __forceinline__ void argmax_unkey(uint64_t key, float& score, int& idx) {
  const uint32_t ord = static_cast<uint32_t>(key >> 32);
  score = __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
  idx = static_cast<int>(~static_cast<uint32_t>(key));
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int C>
__device__ __forceinline__ uint64_t dpp_mov_u64(uint64_t v) {
  const uint32_t lo = dpp_mov<C>(static_cast<uint32_t>(v));
  const uint32_t hi = dpp_mov<C>(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Largest 64-bit key over the wave; every lane returns it. Branch-free: one
// 64-bit compare and two selects per step.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  k = max_u64(k, dpp_mov_u64<kDppXor8>(k));
  k = max_u64(k, dpp_mov_u64<kDppRor4>(k));
  k = max_u64(k, dpp_mov_u64<kDppXor2>(k));
  k = max_u64(k, dpp_mov_u64<kDppXor1>(k));
  const auto plo = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(k), static_cast<uint32_t>(k), false, false);
  const auto phi = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(k >> 32), static_cast<uint32_t>(k >> 32),
                                                    false, false);
  k = max_u64((static_cast<uint64_t>(phi[0]) << 32) | plo[0], (static_cast<uint64_t>(phi[1]) << 32) | plo[1]);
  const auto qlo = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(k), static_cast<uint32_t>(k), false, false);
  const auto qhi = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(k >> 32), static_cast<uint32_t>(k >> 32),
                                                    false, false);
  return max_u64((static_cast<uint64_t>(qhi[0]) << 32) | qlo[0], (static_cast<uint64_t>(qhi[1]) << 32) | qlo[1]);
}

// (score, index) arg-max over the wave, the lowest index winning exact ties;
// every lane returns the winner.
__device__ __forceinline__ void wave_argmax(float& score, int& idx) {
  argmax_unkey(wave_max_u64(argmax_key(score, idx)), score, idx);
}

}  // namespace dg
