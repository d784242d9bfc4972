// Acceptance, renoise and stop of one canvas (the per-canvas half of a
// sampler step), run by accept_renoise_kernel with one workgroup per canvas.
//
// One thread per position, kAcceptThreads (256) positions at most:
//   - only positions with H <= b can come before the last accepted one, so
//     when fewer than 64 have it (every wave counts them from the whole
//     canvas's entropies, which each wave loads), wave 0 sorts those alone
//     (plus the smallest key above b) with the smallest bitonic network that
//     holds them, while the other waves draw the renoise tokens, and a
//     single barrier ends the step; otherwise:
//   - sort the L keys (entropy bits << 32 | position) ascending with a
//     bitonic network, in-wave steps by DPP and permlane swaps (no LDS round
//     trip) and the cross-wave steps through LDS (entropies are >= +0, so
//     their fp32 bit patterns order like the values; equal entropies fall
//     back to position order);
//   - inclusive fp64 scan C_i of the sorted entropies; position i of the
//     order is acceptable while C_i - H_i <= b (H_i is the running maximum of
//     an ascending order), and the accepted set is the longest acceptable
//     prefix ("DiffusionGemma Lab", §2 item 2; boxwrench.dev, Algorithm 1,
//     entropy-bounded acceptance); it is never empty since C_0 - H_0 = 0;
//   - next canvas: the sample where accepted, else a fresh uniform token
//     (boxwrench.dev, Algorithm 1: the remainder is renoised uniformly);
//   - stop = previous argmax given, equal at all positions, and mean entropy
//     below the threshold ("DiffusionGemma Lab", §2 item 3).
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace dg {
namespace accept_detail {

constexpr int kWaves = kAcceptThreads / kWave;

// The 64-bit key of lane (lane ^ j), j a power of two below the wave size
// (a constant once the sorting network is unrolled).
__device__ __forceinline__ uint64_t key_xor(uint64_t v, int j) {
  switch (j) {
    case 1: return lane_xor64<1>(v);
    case 2: return lane_xor64<2>(v);
    case 4: return lane_xor64<4>(v);
    case 8: return lane_xor64<8>(v);
    case 16: return lane_xor64<16>(v);
    default: return lane_xor64<32>(v);
  }
}

// v of lane i - s within its row of 16 lanes (row_shr:s, CTRL = 0x110 + s),
// or 0 where that lane lies before the row.
template <int CTRL>
__device__ __forceinline__ double shifted_in_row(double v) {
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b), CTRL, 0xF, 0xF, false));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(b >> 32), CTRL, 0xF, 0xF, false));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}

__device__ __forceinline__ double read_lane_f64(double v, int lane) {
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(v));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b), lane));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane));
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(hi) << 32) | lo));
}


}  // namespace accept_detail

// Per-thread inputs of accept_canvas, loaded by the caller up front so that
// every load of the kernel is in flight at once: position t's entropy,
// argmax, sample and previous argmax (t < L), the canvas's seed and step,
// and the entropies of positions 4 (t % 64) .. +3, so that every wave holds
// the whole canvas's entropies.
struct AcceptInputs {
  float h = 0.0f;
  int32_t am = 0, smp = 0, prev = 0;
  uint64_t seed = 0;
  int32_t step = 0;
  float hv[4] = {0.0f, 0.0f, 0.0f, 0.0f};   // entropies of positions 4 (t % 64) + i (every wave holds all)
};

// Issues every load accept_canvas needs for thread t of `canvas`.
__device__ __forceinline__ AcceptInputs load_accept_inputs(const AcceptArgs& a, int32_t canvas, int t) {
  AcceptInputs in;
  if (t < a.canvas_len) {
    const int64_t at = static_cast<int64_t>(canvas) * a.canvas_len + t;
    in.h = a.entropy[at];
    in.am = a.argmax[at];
    in.smp = a.sample[at];
    if (a.prev_argmax != nullptr) in.prev = a.prev_argmax[at];
  }
  const int lane = t & (kWave - 1);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = 4 * lane + i;
    if (p < a.canvas_len) in.hv[i] = a.entropy[static_cast<int64_t>(canvas) * a.canvas_len + p];
  }
  in.seed = a.seeds[canvas];
  in.step = a.steps != nullptr ? a.steps[canvas] : a.step;
  return in;
}

// Runs the acceptance of `canvas` on a workgroup of NT threads (NT a multiple
// of 64, at least kAcceptThreads); threads from kAcceptThreads on only join
// the barriers. Every thread of the workgroup must call it, with its inputs
// from load_accept_inputs.
template <int NT>
__device__ __forceinline__ void accept_canvas(const AcceptArgs& a, int32_t canvas, const AcceptInputs& in) {
  using namespace accept_detail;
  static_assert(NT % kWave == 0 && NT >= kAcceptThreads, "accept_canvas: bad workgroup size");
  __shared__ uint64_t s_key[kAcceptThreads];
  __shared__ double s_wsum[kWaves];
  __shared__ double s_hsum[kWaves];
  __shared__ int32_t s_same[kWaves];
  __shared__ int32_t s_wmin[kWaves];
  __shared__ uint8_t s_acc[kAcceptThreads];
  __shared__ int32_t s_ren[kWave];
  __shared__ int32_t s_kstar;

  const int tid = threadIdx.x;
  const bool part = tid < kAcceptThreads;   // owns a key slot
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int32_t L = a.canvas_len;
  const int64_t base = static_cast<int64_t>(canvas) * L;
  const bool valid = tid < L;
  const float h = in.h;
  const int32_t am = in.am, smp = in.smp;

  // Independent of the order: mean entropy (fp64, in position order) and
  // argmax stability, published by the last barrier of either path.
  double hsum = valid ? static_cast<double>(h) : 0.0;
  hsum = wave_sum(hsum);
  const bool same = !valid || (a.prev_argmax != nullptr && in.prev == am);
  const bool wave_same = __builtin_amdgcn_ballot_w64(!same) == 0;
  if (part && lane == 0) {
    s_hsum[wave] = hsum;
    s_same[wave] = wave_same ? 1 : 0;
  }
  auto renoise_of = [&](int pos) -> int32_t {
    const Words4 rw = philox4x32_10(0u, static_cast<uint32_t>(pos), static_cast<uint32_t>(in.step),
                                    kTagRenoise, static_cast<uint32_t>(in.seed),
                                    static_cast<uint32_t>(in.seed >> 32));
    return uniform_token(rw.w[0], static_cast<uint32_t>(a.vocab));
  };
  // Only entropies <= b can precede the last accepted position: the
  // exclusive prefix sum before sorted rank r is at least the entropy at rank
  // r - 1. So the accepted set is a prefix of the sorted set C = {H <= b},
  // followed at most by the smallest key outside C. Every wave counts C from
  // the canvas-wide entropies it holds, so all of them take the same path
  // without a barrier. When C holds fewer than 64 positions (all but the last
  // steps of a run), wave 0 sorts C alone while the other waves draw the
  // renoise tokens, and one barrier ends the step; its scan is the full
  // sort's first-wave scan, so both paths give the same bits. Otherwise the
  // whole canvas is sorted.
  uint64_t cball[4];
  int32_t n_c = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int p = 4 * lane + i;
    cball[i] = __builtin_amdgcn_ballot_w64(p < L && in.hv[i] <= a.bound);
    n_c += __builtin_popcountll(cball[i]);
  }
  int32_t kstar;
  int32_t renoise = 0;
  if (n_c < kWave) {
    if (wave == 0) {
      // lanes 0..n_c-1: C's keys (placed through LDS by this wave alone);
      // lane n_c: the smallest key outside C (all of C's keys are below it);
      // the rest empty
      uint64_t outside = ~0ull;
      int32_t off = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int p = 4 * lane + i;
        const uint64_t k = (static_cast<uint64_t>(__float_as_uint(in.hv[i])) << 32) | static_cast<uint32_t>(p);
        const bool in_c = ((cball[i] >> lane) & 1) != 0;
        if (in_c) {
          const int below = __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(cball[i] >> 32),
                                                      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(cball[i]), 0));
          s_key[off + below] = k;
        } else if (p < L) {
          outside = k < outside ? k : outside;
        }
        off += __builtin_popcountll(cball[i]);
        if (p < kAcceptThreads) s_acc[p] = 0;
      }
      const uint64_t omin = ~wave_max_u64(~outside);
      uint64_t k2 = lane < n_c ? s_key[lane] : (lane == n_c ? omin : ~0ull);
      // bitonic sort of the first m lanes, m the smallest power of two above
      // n_c (lanes m.. hold empty keys, so the result is the full network's)
      const int m = n_c == 0 ? 1 : 1 << (32 - __builtin_clz(static_cast<uint32_t>(n_c)));
#pragma unroll
      for (int k = 2; k <= kWave; k <<= 1) {
        if (k > m) break;
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1) {
          const uint64_t other = key_xor(k2, j);
          const bool ascending = (lane & k) == 0;
          const bool lower = (lane & j) == 0;
          const uint64_t lo = k2 < other ? k2 : other;
          const uint64_t hi = k2 < other ? other : k2;
          k2 = (lower == ascending) ? lo : hi;
        }
      }
      const bool real = k2 != ~0ull;
      const double hs = real ? static_cast<double>(__uint_as_float(static_cast<uint32_t>(k2 >> 32))) : 0.0;
      double incl = hs;
      incl += shifted_in_row<0x111>(incl);
      incl += shifted_in_row<0x112>(incl);
      incl += shifted_in_row<0x114>(incl);
      incl += shifted_in_row<0x118>(incl);
      {
        const double t0 = read_lane_f64(incl, 15), t1 = read_lane_f64(incl, 31), t2 = read_lane_f64(incl, 47);
        const int row = lane >> 4;
        incl += row == 0 ? 0.0 : row == 1 ? t0 : row == 2 ? t0 + t1 : (t0 + t1) + t2;
      }
      const bool ok = real && (incl - hs) <= static_cast<double>(a.bound);
      // the rank after the smallest key outside C (rank n_c + 1, which may lie
      // past the last lane) is never acceptable: its prefix holds an entropy
      // above b; nor is an empty lane
      int32_t first_bad = (real && !ok) || !real ? lane : L;
      first_bad = wave_min_int(first_bad);
      const int32_t ks = min(first_bad, min(n_c + 1, L));
      if (real && lane < ks) s_acc[static_cast<uint32_t>(k2)] = 1;
      if (lane == 0) s_kstar = ks;
    } else {
      // the renoise tokens: each wave its own positions, wave 1 also wave 0's
      if (valid) renoise = renoise_of(tid);
      if (wave == 1 && lane < L) s_ren[lane] = renoise_of(lane);
    }
    __syncthreads();
    if (wave == 0 && valid) renoise = s_ren[lane];
    kstar = s_kstar;
  } else {
    if (valid) renoise = renoise_of(tid);
    uint64_t key = valid ? ((static_cast<uint64_t>(__float_as_uint(h)) << 32) | static_cast<uint32_t>(tid))
                         : ~0ull;
    if (part) s_acc[tid] = 0;
    // bitonic sort of 256 keys, ascending. Compare-exchange partners closer
    // than a wave are reached with lane shuffles; only the three steps whose
    // partner lies in another wave go through LDS.
#pragma unroll
    for (int k = 2; k <= kAcceptThreads; k <<= 1) {
#pragma unroll
      for (int j = k >> 1; j > 0; j >>= 1) {
        uint64_t other;
        if (j >= kWave) {
          if (part) s_key[tid] = key;
          __syncthreads();
          other = part ? s_key[tid ^ j] : key;
          __syncthreads();
        } else {
          other = key_xor(key, j);
        }
        const bool ascending = (tid & k) == 0;
        const bool lower = (tid & j) == 0;
        const uint64_t lo = key < other ? key : other;
        const uint64_t hi = key < other ? other : key;
        key = (lower == ascending) ? lo : hi;
      }
    }

    // inclusive fp64 scan of sorted entropies: rows of 16 lanes by DPP shifts,
    // then row offsets, then wave offsets
    const double hs = valid ? static_cast<double>(__uint_as_float(static_cast<uint32_t>(key >> 32))) : 0.0;
    double incl = hs;
    incl += shifted_in_row<0x111>(incl);
    incl += shifted_in_row<0x112>(incl);
    incl += shifted_in_row<0x114>(incl);
    incl += shifted_in_row<0x118>(incl);
    {
      const double t0 = read_lane_f64(incl, 15), t1 = read_lane_f64(incl, 31), t2 = read_lane_f64(incl, 47);
      const int row = lane >> 4;
      incl += row == 0 ? 0.0 : row == 1 ? t0 : row == 2 ? t0 + t1 : (t0 + t1) + t2;
    }
    if (part && lane == kWave - 1) s_wsum[wave] = incl;
    __syncthreads();
    for (int w = 0; w < wave && w < kWaves; ++w) incl += s_wsum[w];

    // first sorted index that is not acceptable; k* = that index (or L)
    const bool ok = valid && (incl - hs) <= static_cast<double>(a.bound);
    int32_t first_bad = (valid && !ok) ? tid : L;
    first_bad = wave_min_int(first_bad);
    __syncthreads();
    if (part && lane == 0) s_wmin[wave] = first_bad;
    __syncthreads();
    kstar = s_wmin[0];
    for (int w = 1; w < kWaves; ++w) kstar = min(kstar, s_wmin[w]);
    if (valid) s_acc[static_cast<uint32_t>(key)] = static_cast<uint8_t>(tid < kstar);
    __syncthreads();  // accept flags scattered by position
  }
  double total = 0.0;
  int all_same = 1;
  for (int w = 0; w < kWaves; ++w) {
    total += s_hsum[w];
    all_same &= s_same[w];
  }
  const double mean_h = total / static_cast<double>(L);

  if (valid) {
    const bool accepted = s_acc[tid] != 0;
    a.canvas_out[base + tid] = accepted ? smp : renoise;
    if (a.accept_out) a.accept_out[base + tid] = accepted ? 1 : 0;
    if (a.argmax_out) a.argmax_out[base + tid] = am;
    if (a.sample_out) a.sample_out[base + tid] = smp;
    if (a.entropy_out) a.entropy_out[base + tid] = h;
  }
  if (tid == 0) {
    const bool stop = a.prev_argmax != nullptr && all_same &&
                      mean_h < static_cast<double>(a.stop_mean_entropy);
    if (a.n_accept_out) a.n_accept_out[canvas] = kstar;
    if (a.mean_entropy_out) a.mean_entropy_out[canvas] = static_cast<float>(mean_h);
    if (a.stop_out) a.stop_out[canvas] = stop ? 1 : 0;
    if (a.run_active) {
      a.run_steps_used[canvas] = a.step + 1;
      a.run_temperature[canvas] = a.run_next_temperature;
      if (stop) {
        a.run_stopped[canvas] = 1;
        a.run_active[canvas] = 0;
      }
    }
  }
}

}  // namespace dg
