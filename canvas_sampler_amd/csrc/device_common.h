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
// per lane (bf16) so every load is fully coalesced. A supergroup is 64
// consecutive stripes; block j = 64*supergroup + slot gathers one slot across
// the 64 stripes, so a lane of a wave streaming a supergroup owns exactly one
// block and never needs another lane to finish it.
constexpr int kSlotIds = 8;
constexpr int kSlots = 64;
constexpr int kStripeIds = kSlotIds * kSlots;        // 512
constexpr int kStripesPerSg = 64;
constexpr int kSgIds = kStripeIds * kStripesPerSg;   // 32768

// Counter word 3 of each random draw.
constexpr uint32_t kTagInit = 0;
constexpr uint32_t kTagBlock = 1;
constexpr uint32_t kTagElem = 2;
constexpr uint32_t kTagRenoise = 3;

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

// ---- wave64 reductions (butterfly over all 64 lanes) ----
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// (score, index) arg-max with the lowest index winning exact ties.
__device__ __forceinline__ void wave_argmax(float& score, int& idx) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float s2 = __shfl_xor(score, o, kWave);
    const int i2 = __shfl_xor(idx, o, kWave);
    if (s2 > score || (s2 == score && i2 < idx)) {
      score = s2;
      idx = i2;
    }
  }
}

}  // namespace dg
