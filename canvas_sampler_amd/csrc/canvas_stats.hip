// canvas_stats_kernel: the streaming pass of one sampler step.
//
// For every row (one canvas position) of z = logits it computes, in one read
// of the row from HBM:
//   - the entropy in nats of softmax(z/T) ("DiffusionGemma Lab", §2 item 2:
//     positions are ranked by entropy; item 4: the temperature sharpens the
//     distribution), from an online maximum and the two sums
//     S = sum 2^t and W = sum t*2^t with t = (z - ref)*log2(e)/T, so that
//     H = ln 2 * (log2 S - W/S);
//   - the argmax of the raw logits, lowest id on ties (§2 item 5: the argmax
//     canvas is the output);
//   - one multinomial sample (§2 item 5) by the two-level Gumbel-max protocol:
//     each lane owns one block per supergroup (one 8-id slot across 64
//     stripes), forms that block's log-sum-exp on the fly and adds its block
//     Gumbel; the best block j* is re-read (512 ids, 0.2% of the row) and the
//     sample is the id of j* with the largest z/T + element Gumbel.
//
// Layout and schedule (gfx950, wave64): rows are V-contiguous. A workgroup of
// eight waves handles a row (or one split of it); its waves take 32768-id
// supergroups round-robin. Each lane issues one 16-byte load per 512-id stripe
// (bf16; two for fp32), so a wave's load covers 1 KiB (bf16) or 2 KiB (fp32)
// of consecutive memory. Loads are raw buffer loads on a per-row resource
// (hardware range check, no branches), marked non-temporal, and a register
// ring keeps two batches of 8 stripes in flight while a third is reduced.
// Per element the loop costs one convert, half a max, one fma, one v_exp_f32,
// one add and one fma; per-block work is amortised over 512 ids per lane.
// When its stream ends, each wave resolves its own exact argmax (the lanes
// holding the wave maximum re-read the batch where they first saw it) and
// resamples its own best block, overlapping other waves still streaming; the
// workgroup then merges eight 32-byte partials. A row split over several
// workgroups (for very short batches) is merged by the last workgroup to
// finish (atomic ticket, release/acquire at agent scope).
#include "device_common.h"
#include "kernels.h"

namespace dg {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.69314718055994530942;
constexpr int kWaves = kStatsThreads / kWave;
constexpr float kNegInf = -__builtin_inff();

// The running reference trails the true maximum by up to 8 (log2 units, a
// factor 256) before the sums are rescaled.
constexpr float kRefSlack = 8.0f;

// Offset used for prefetches past a wave's last batch: beyond every row
// resource (rows hold fewer than 2^31 - 2^16 bytes) even with the largest
// immediate offset added, so those loads return zero and read nothing.
constexpr uint32_t kPastEnd = 0x7FFF0000u;

// Cache policy of the streaming loads: non-temporal (each logit is read once).
constexpr int kStreamPolicy = 2;


template <bool kBf16>
struct Geometry {
  static constexpr int kLoadsPerStripe = kBf16 ? 1 : 2;   // 16-byte loads per lane
  static constexpr int kElemBytes = kBf16 ? 2 : 4;
};

// Loads NB stripes of the lane's slot with raw buffer loads on the row's
// resource (base = row start, size = V elements): `byte0` is the byte offset of
// the lane's chunk in the batch's first stripe. The loads are unconditional;
// bytes past V read as zero (hardware range check) and are masked by the
// caller, so no load sits behind a branch and the next batch stays in flight
// while the current one is reduced.
template <bool kBf16, int NB>
__device__ __forceinline__ void load_batch(uint4 (&buf)[NB * Geometry<kBf16>::kLoadsPerStripe],
                                           __amdgpu_buffer_rsrc_t rsrc, uint32_t byte0) {
  constexpr int LPS = Geometry<kBf16>::kLoadsPerStripe;
  constexpr int kEB = Geometry<kBf16>::kElemBytes;
#pragma unroll
  for (int s = 0; s < NB; ++s) {
#pragma unroll
    for (int h = 0; h < LPS; ++h) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(
          rsrc, static_cast<int>(byte0 + static_cast<uint32_t>((s * kStripeIds + h * 4) * kEB)), 0,
          kStreamPolicy);
      buf[s * LPS + h] = make_uint4(v[0], v[1], v[2], v[3]);
    }
  }
}

// Widens a loaded batch to fp32: z[s*8 + e] is id id0 + s*512 + e.
template <bool kBf16, int NB>
__device__ __forceinline__ void unpack_batch(const uint4 (&buf)[NB * Geometry<kBf16>::kLoadsPerStripe],
                                             float (&z)[NB * kSlotIds]) {
#pragma unroll
  for (int s = 0; s < NB; ++s) {
    if constexpr (kBf16) {
      const uint4 q = buf[s];
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        z[s * 8 + 2 * i] = __uint_as_float(w[i] << 16);
        z[s * 8 + 2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 q = buf[2 * s + h];
        z[s * 8 + 4 * h + 0] = __uint_as_float(q.x);
        z[s * 8 + 4 * h + 1] = __uint_as_float(q.y);
        z[s * 8 + 4 * h + 2] = __uint_as_float(q.z);
        z[s * 8 + 4 * h + 3] = __uint_as_float(q.w);
      }
    }
  }
}

// active[canvas] read through the aligned 32-bit word that holds it, so that
// the workgroup-uniform read is a scalar load and does not queue behind the
// vector loads already in flight (the word lies in the same page as the byte).
__device__ __forceinline__ bool active_flag(const uint8_t* active, int32_t canvas) {
  const uint32_t mis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(active) & 3);
  const uint32_t* words = reinterpret_cast<const uint32_t*>(active - mis);
  const uint32_t at = static_cast<uint32_t>(canvas) + mis;
  return ((words[at >> 2] >> (8 * (at & 3))) & 0xFFu) != 0;
}

// Per-lane running state of the pass. The current block's sums stay in fp32
// (at most 512 ids per lane, each term below 2^8 relative to ref) and are
// folded into the fp64 row sums when the block ends.
struct LaneState {
  double s = 0.0;        // sum 2^t over finished blocks, relative to ref
  double w = 0.0;        // sum t*2^t over finished blocks, relative to ref
  float sb = 0.f;        // current block's sum 2^t, relative to ref
  float wb = 0.f;        // current block's sum t*2^t, relative to ref
  float ref = kNegInf;   // reference, <= max z*c seen so far
  float m = kNegInf;     // max raw logit
  int32_t search = 0x7FFFFFFF;  // first id of the batch where m was first seen
  float best = kNegInf;  // best block score (log2 units)
  int32_t bestj = 0x7FFFFFFF;  // its block; the lowest one among equal scores
};

// Sums of 2^t and t*2^t over a batch held in z: four interleaved fma chains
// for t*2^t, then an in-place halving tree for 2^t. A -inf logit gives
// 2^t = 0 but t*2^t = 0 * -inf = NaN; the rare batch where that happens
// recomputes t*2^t from the stored 2^t (t = log2 2^t wherever 2^t > 0), so
// the logits themselves need not stay live after the exponentials.
template <int N>
__device__ __forceinline__ void batch_sums(const float (&z)[N], float c, float ref, float& bs,
                                           float& bw) {
  float e[N];
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const float t = fmaf(z[k], c, -ref);
    e[k] = __builtin_amdgcn_exp2f(t);
    acc[k & 3] = fmaf(t, e[k], acc[k & 3]);
  }
  bw = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  if (bw != bw) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = 0.f;
#pragma unroll
    for (int k = 0; k < N; ++k)
      if (e[k] > 0.f) acc[k & 3] = fmaf(__log2f(e[k]), e[k], acc[k & 3]);
    bw = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  }
#pragma unroll
  for (int h = N / 2; h >= 1; h >>= 1) {
#pragma unroll
    for (int i = 0; i < h; ++i) e[i] = e[i] + e[i + h];
  }
  bs = e[0];
}

// 2^d for a reference shift d <= 0 (exact in double): the factor only scales
// partial sums, so fp32 v_exp_f32 of the rounded shift is accurate enough
// (relative error below 1e-6 wherever the factor is not negligible).
__device__ __forceinline__ double scale_of(double d) {
  return static_cast<double>(__builtin_amdgcn_exp2f(static_cast<float>(d)));
}

// Rescales a lane's sums from reference st.ref to the larger reference r.
__device__ __forceinline__ void rebase(LaneState& st, float r) {
  if (st.ref != kNegInf) {
    const double d = static_cast<double>(st.ref) - static_cast<double>(r);
    const double f = scale_of(d);
    st.w = f * (st.w + d * st.s);
    st.s *= f;
    const float ff = static_cast<float>(f), df = static_cast<float>(d);
    st.wb = ff * (st.wb + df * st.sb);
    st.sb *= ff;
  }
  st.ref = r;
}

// Chunk-ordered reduction of a batch against reference ref: for every
// 8-id chunk, widen, 2^t with t = z*c - ref, the chunk's fma chain for t*2^t,
// an 8-way tree for 2^t and a max. Written chunk by chunk so that each chunk's
// work can start when its own load has landed. Returns the batch maximum;
// bs, bw as in batch_sums (a -inf logit gives NaN in bw; see there).
template <bool kBf16, int NB>
__device__ __forceinline__ float chunked_sums(const uint4 (&buf)[NB * Geometry<kBf16>::kLoadsPerStripe],
                                              float c, float ref, float& bs, float& bw) {
  float cs[NB];
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float bm = kNegInf;
#pragma unroll
  for (int s = 0; s < NB; ++s) {
    float zz[kSlotIds];
    if constexpr (kBf16) {
      const uint4 q = buf[s];
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        zz[2 * i] = __uint_as_float(w[i] << 16);
        zz[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 q = buf[2 * s + h];
        zz[4 * h + 0] = __uint_as_float(q.x);
        zz[4 * h + 1] = __uint_as_float(q.y);
        zz[4 * h + 2] = __uint_as_float(q.z);
        zz[4 * h + 3] = __uint_as_float(q.w);
      }
    }
    float e[kSlotIds];
#pragma unroll
    for (int k = 0; k < kSlotIds; ++k) {
      const float t = fmaf(zz[k], c, -ref);
      e[k] = __builtin_amdgcn_exp2f(t);
      acc[k & 3] = fmaf(t, e[k], acc[k & 3]);
    }
    bm = max3_raw(bm, max3_raw(zz[0], zz[1], zz[2]),
                  max3_raw(max3_raw(zz[3], zz[4], zz[5]), zz[6], zz[7]));
    cs[s] = ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
  }
#pragma unroll
  for (int h = NB / 2; h >= 1; h >>= 1) {
#pragma unroll
    for (int i = 0; i < h; ++i) cs[i] = cs[i] + cs[i + h];
  }
  bs = cs[0];
  bw = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  return bm;
}

// Reduces one batch on the slow path: for a lane that has seen no finite
// logit yet, whose batch holds -inf logits (2^t = 0 but t*2^t = 0 * -inf =
// NaN), whose maximum jumped past the lag bound, or for the batch that
// crosses V (ids past V masked to -inf). The widened batch gives the batch
// maximum first, the reference moves up if needed, and the sums are formed
// against it.
template <bool kBf16, int NB>
__device__ __forceinline__ void slow_batch(const uint4 (&buf)[NB * Geometry<kBf16>::kLoadsPerStripe],
                                           int64_t id0, int32_t vocab, float c, bool tail,
                                           LaneState& st) {
  float z[NB * kSlotIds];
  unpack_batch<kBf16, NB>(buf, z);
  if (tail) {
#pragma unroll
    for (int s = 0; s < NB; ++s)
#pragma unroll
      for (int e = 0; e < kSlotIds; ++e)
        if (id0 + s * kStripeIds + e >= vocab) z[s * 8 + e] = kNegInf;
  }
  float bm = z[0];
#pragma unroll
  for (int k = 1; k < NB * kSlotIds; ++k) bm = fmaxf(bm, z[k]);
  if (bm == kNegInf) return;
  const float bref = __fmul_rn(bm, c);
  if (st.ref == kNegInf || bref > st.ref + kRefSlack) rebase(st, bref);
  float bs, bw;
  batch_sums<NB * kSlotIds>(z, c, st.ref, bs, bw);
  st.sb += bs;
  st.wb += bw;
}

// Reduces one complete batch (every id below V) into the lane state. The
// exponentials use the reference of the batches before (it lags the running
// maximum), so each chunk is reduced as soon as its load lands instead of
// after a batch-wide maximum; the batch maximum is folded in afterwards. A
// lag of up to 2^64 cannot overflow fp32; the rare batches that need more go
// to the slow path, behind a wave-uniform branch.
template <bool kBf16, int NB>
__device__ __forceinline__ void fast_batch(const uint4 (&buf)[NB * Geometry<kBf16>::kLoadsPerStripe],
                                           int64_t batch_first_id, int64_t id0, int32_t vocab, float c,
                                           LaneState& st) {
  constexpr float kMaxLag = 64.0f;
  float bs, bw;
  const float bm = chunked_sums<kBf16, NB>(buf, c, st.ref, bs, bw);
  // exact argmax bookkeeping: first batch that attains the lane's maximum
  if (bm > st.m) {
    st.m = bm;
    st.search = static_cast<int32_t>(batch_first_id);
  }
  const float bref = __fmul_rn(bm, c);
  const bool bad = !(bw == bw) || !(bref <= st.ref + kMaxLag);  // NaN, fresh lane, or a big jump
  if (__builtin_amdgcn_ballot_w64(bad) != 0 && bad) {
    slow_batch<kBf16, NB>(buf, id0, vocab, c, false, st);
  } else {
    st.sb += bs;
    st.wb += bw;
  }
  const bool lift = bref > st.ref + kRefSlack;
  if (__builtin_amdgcn_ballot_w64(lift) != 0 && lift) rebase(st, bref);
}

// Merges partial b into a: entropy sums, argmax (lowest id among equal
// maxima) and the sample of the best block (lowest block among equal scores).
__device__ __forceinline__ void merge_partial(RowPartial& a, const RowPartial& b) {
  if (b.m > a.m || (b.m == a.m && b.argmax < a.argmax)) {
    a.m = b.m;
    a.argmax = b.argmax;
  }
  if (b.best > a.best || (b.best == a.best && b.bestj < a.bestj)) {
    a.best = b.best;
    a.bestj = b.bestj;
    a.sample = b.sample;
  }
  if (b.ref == kNegInf) return;
  if (a.ref == kNegInf) {
    a.ref = b.ref;
    a.s = b.s;
    a.w = b.w;
    return;
  }
  const float r = fmaxf(a.ref, b.ref);
  const double da = static_cast<double>(a.ref) - static_cast<double>(r);
  const double db = static_cast<double>(b.ref) - static_cast<double>(r);
  const double fa = scale_of(da), fb = scale_of(db);
  a.w = fa * (a.w + da * a.s) + fb * (b.w + db * b.s);
  a.s = fa * a.s + fb * b.s;
  a.ref = r;
}

// The partial held by lane (lane ^ J).
template <int J>
__device__ __forceinline__ RowPartial partial_xor(const RowPartial& p) {
  RowPartial q;
  q.s = __longlong_as_double(static_cast<long long>(lane_xor64<J>(static_cast<uint64_t>(__double_as_longlong(p.s)))));
  q.w = __longlong_as_double(static_cast<long long>(lane_xor64<J>(static_cast<uint64_t>(__double_as_longlong(p.w)))));
  q.ref = __uint_as_float(lane_xor<J>(__float_as_uint(p.ref)));
  q.m = __uint_as_float(lane_xor<J>(__float_as_uint(p.m)));
  q.argmax = static_cast<int32_t>(lane_xor<J>(static_cast<uint32_t>(p.argmax)));
  q.best = __uint_as_float(lane_xor<J>(__float_as_uint(p.best)));
  q.bestj = static_cast<int32_t>(lane_xor<J>(static_cast<uint32_t>(p.bestj)));
  q.sample = static_cast<int32_t>(lane_xor<J>(static_cast<uint32_t>(p.sample)));
  return q;
}

// Finishes a wave once its stream ends, while other waves may still be
// streaming: reduces the lane states to one partial, finds the exact first id
// of the wave's maximum (the lanes holding it re-read the batch where they
// first saw it), and draws the in-block sample of the wave's best block (lane
// k reads the block's 8 ids in stripe k). Both re-reads are issued together,
// before any dependent work. Returns the partial in every lane.
template <bool kBf16, int NB>
__device__ __forceinline__ RowPartial wave_finish(const LaneState& st, __amdgpu_buffer_rsrc_t rsrc,
                                                  int32_t vocab, float temp, int32_t pos, int32_t step,
                                                  uint32_t k0, uint32_t k1, int lane) {
  constexpr int LPS = Geometry<kBf16>::kLoadsPerStripe;
  constexpr uint32_t kEB = Geometry<kBf16>::kElemBytes;
  RowPartial p;
  p.m = wave_max(st.m);
  float bscore = st.best;
  int32_t bj = st.bestj;
  wave_argmax(bscore, bj);
  p.best = bscore;
  p.bestj = bj;

  // loads: this lane's batch if it holds the wave maximum, and stripe `lane`
  // of the best block (offsets past the resource read nothing)
  const bool holds_max = p.m != kNegInf && st.m == p.m;
  uint4 mine[NB * LPS];
  load_batch<kBf16, NB>(mine, rsrc,
                        holds_max ? static_cast<uint32_t>(st.search + lane * kSlotIds) * kEB : kPastEnd);
  const int64_t v0 = static_cast<int64_t>(bj >> 6) * kSgIds + static_cast<int64_t>(lane) * kStripeIds +
                     (bj & 63) * kSlotIds;
  const bool block_ok = bscore != kNegInf && v0 < vocab;
  uint4 blk[LPS];
#pragma unroll
  for (int h = 0; h < LPS; ++h) {
    const uint32_t off = block_ok ? static_cast<uint32_t>(v0 + 4 * h) * kEB : kPastEnd;
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, static_cast<int>(off), 0, 0);
    blk[h] = make_uint4(v[0], v[1], v[2], v[3]);
  }

  // entropy sums (independent of the loads); every block has been folded
  const float r = wave_max(st.ref);
  double s = 0.0, w = 0.0;
  if (st.ref != kNegInf) {
    const double d = static_cast<double>(st.ref) - static_cast<double>(r);
    const double f = scale_of(d);
    s = f * st.s;
    w = f * (st.w + d * st.s);
  }
  p.s = wave_sum(s);
  p.w = wave_sum(w);
  p.ref = r;
  // element Gumbel noise of this lane's 8 block ids: words of (v0>>2) and
  // (v0>>2)+1 (v0 is a multiple of 8: word e belongs to id v0 + e); it needs
  // only the block index, so it is formed while the re-reads are in flight
  const Words4 g0 = philox4x32_10(static_cast<uint32_t>(v0 >> 2), static_cast<uint32_t>(pos),
                                  static_cast<uint32_t>(step), kTagElem, k0, k1);
  const Words4 g1 = philox4x32_10(static_cast<uint32_t>(v0 >> 2) + 1u, static_cast<uint32_t>(pos),
                                  static_cast<uint32_t>(step), kTagElem, k0, k1);
  const uint32_t words[8] = {g0.w[0], g0.w[1], g0.w[2], g0.w[3], g1.w[0], g1.w[1], g1.w[2], g1.w[3]};
  float gum[kSlotIds];
#pragma unroll
  for (int e = 0; e < kSlotIds; ++e) gum[e] = gumbel(words[e]);
  __builtin_amdgcn_sched_barrier(0);

  // exact argmax of the wave: lowest id equal to the maximum
  int32_t cand = 0x7FFFFFFF;
  if (holds_max) {
    float z[NB * kSlotIds];
    unpack_batch<kBf16, NB>(mine, z);
#pragma unroll
    for (int k = NB * kSlotIds - 1; k >= 0; --k) {  // ids increase with k
      const int64_t id = static_cast<int64_t>(st.search) + lane * kSlotIds + (k >> 3) * kStripeIds + (k & 7);
      if (id < vocab && z[k] == p.m) cand = static_cast<int32_t>(id);
    }
  }
  p.argmax = wave_min_int(cand);

  // in-block resample of the wave's best block: z/T as z * (1/T), within an
  // ulp of the quotient
  const float inv_t = 1.0f / temp;
  float best = kNegInf;
  int32_t best_id = 0x7FFFFFFF;
  if (block_ok) {
    float zb[kSlotIds];
    if constexpr (kBf16) {
      const uint32_t w4[4] = {blk[0].x, blk[0].y, blk[0].z, blk[0].w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        zb[2 * q] = __uint_as_float(w4[q] << 16);
        zb[2 * q + 1] = __uint_as_float(w4[q] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        zb[4 * h + 0] = __uint_as_float(blk[h].x);
        zb[4 * h + 1] = __uint_as_float(blk[h].y);
        zb[4 * h + 2] = __uint_as_float(blk[h].z);
        zb[4 * h + 3] = __uint_as_float(blk[h].w);
      }
    }
#pragma unroll
    for (int e = 0; e < kSlotIds; ++e) {
      if (v0 + e < vocab) {
        const float score = zb[e] * inv_t + gum[e];
        if (score > best) {  // ids increase with e: strict > keeps the lower
          best = score;
          best_id = static_cast<int32_t>(v0 + e);
        }
      }
    }
  }
  wave_argmax(best, best_id);
  p.sample = best_id;
  return p;
}

// Writes a row's outputs from its merged partial: H = ln 2 (log2 S - W/S).
__device__ __forceinline__ void row_output(const StatsArgs& a, int32_t r, const RowPartial& p) {
  const double h = kLn2 * (log2(p.s) - p.w / p.s);
  const float hf = static_cast<float>(h);
  a.entropy[r] = hf > 0.0f ? hf : 0.0f;
  a.argmax[r] = p.argmax;
  a.sample[r] = p.sample;
}

// Merges the eight wave partials in a three-level tree across lanes 0..7 of
// wave 0 (lane l starts from partial l mod 8); lane 0 returns all eight.
__device__ __forceinline__ RowPartial merge_waves(const RowPartial* s_part, int lane) {
  RowPartial p = s_part[lane & (kWaves - 1)];
  merge_partial(p, partial_xor<4>(p));
  merge_partial(p, partial_xor<2>(p));
  merge_partial(p, partial_xor<1>(p));
  return p;
}

// NB stripes per batch; DEPTH batches in the register ring (DEPTH - 1 in
// flight while one is reduced).
template <bool kBf16, int NB, int DEPTH>
__global__ __launch_bounds__(kStatsThreads) void canvas_stats_kernel(StatsArgs a) {
  constexpr int LPS = Geometry<kBf16>::kLoadsPerStripe;
  constexpr int kBatchesPerSg = kStripesPerSg / NB;
  static_assert(kBatchesPerSg % DEPTH == 0, "the ring must divide a supergroup's batches");
  __shared__ RowPartial s_part[kWaves];

  const int32_t r = static_cast<int32_t>(blockIdx.x) / a.nsplit;
  const int32_t split = static_cast<int32_t>(blockIdx.x) % a.nsplit;
  const int32_t canvas = r / a.canvas_len;
  const int32_t pos = r % a.canvas_len;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave index as a scalar, so the batch loop below is uniform control flow
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int32_t vocab = a.vocab;
  const char* __restrict__ row =
      static_cast<const char*>(a.logits) + static_cast<int64_t>(r) * a.row_stride * Geometry<kBf16>::kElemBytes;

  // The resource covers the row rounded up to 16 bytes (inside the row
  // stride): the range check works per dword, and a dword holding the last
  // bf16 id and one padding id must still be read. Ids past V are masked.
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<char*>(row), 0, ((vocab * Geometry<kBf16>::kElemBytes + 15) / 16) * 16, 0x00020000);
  constexpr uint32_t kEB = Geometry<kBf16>::kElemBytes;
  const uint32_t lane_bytes = static_cast<uint32_t>(lane * kSlotIds) * kEB;

  const int32_t nsg = (vocab + kSgIds - 1) / kSgIds;
  const int32_t sg_begin = static_cast<int32_t>((static_cast<int64_t>(split) * nsg) / a.nsplit);
  const int32_t sg_end = static_cast<int32_t>((static_cast<int64_t>(split + 1) * nsg) / a.nsplit);

  // The two waves sharing a SIMD (w and w + 4) form a pair that streams
  // supergroups sg_begin + w, + 4, ... in batches of NB stripes. Only the
  // row's last supergroup can be partial, and it is the pair's last, so the
  // pair's live batches form a flat range [0, npair): batch b lies in
  // supergroup sg_of(b) at stripe (b % kBatchesPerSg) * NB. The older wave
  // takes the first kFirstShare/16 of that range and the younger one the
  // rest: the SIMD arbiter favours the older wave, and with equal halves the
  // younger one would stream on alone for the last fifth. A supergroup cut
  // by the split is closed in two pieces that the pair combines in LDS.
  // Batches [b_lo, n_fast) of a wave lie wholly below V; the batch that
  // crosses V, if any, is the pair's last.
  constexpr int32_t kFirstShare = 10;
  const int pair = wave & 3;
  const int second = wave >> 2;
  const int32_t pair_sgs = (sg_end - sg_begin - pair + 3) / 4;
  auto sg_of = [&](int32_t b) { return sg_begin + pair + (b / kBatchesPerSg) * 4; };
  auto first_id = [&](int32_t b) {
    return static_cast<int64_t>(sg_of(b)) * kSgIds +
           static_cast<int64_t>(b % kBatchesPerSg) * NB * kStripeIds;
  };
  int32_t npair = 0;
  if (pair_sgs > 0) {
    const int64_t last_sg_first = static_cast<int64_t>(sg_begin + pair + (pair_sgs - 1) * 4) * kSgIds;
    const int64_t left = static_cast<int64_t>(vocab) - last_sg_first;  // > 0
    const int64_t live_last = (left + NB * kStripeIds - 1) / (NB * kStripeIds);
    npair = (pair_sgs - 1) * kBatchesPerSg +
            static_cast<int32_t>(live_last < kBatchesPerSg ? live_last : kBatchesPerSg);
  }
  const int32_t psplit = (npair * kFirstShare / 16) / DEPTH * DEPTH;
  const int32_t b_lo = second ? psplit : 0;
  const int32_t n = second ? npair : psplit;
  const int32_t n_fast = (n > b_lo && first_id(n - 1) + NB * kStripeIds > vocab) ? n - 1 : n;
  const bool cut = psplit % kBatchesPerSg != 0;  // a supergroup is shared by the pair
  const int32_t sg_cut = cut ? sg_of(psplit) : -1;
  // Byte offset of batch b for this lane; batches from n_fast on point beyond
  // the resource, where buffer loads return zero without touching memory, so
  // every prefetch can be issued unconditionally (a load behind a branch would
  // make the compiler wait for it before reducing the current batch).
  auto byte_of = [&](int32_t b) {
    return b < n_fast ? static_cast<uint32_t>(first_id(b)) * kEB + lane_bytes : kPastEnd;
  };

  // Register ring of DEPTH batches. The first loads go out before the per-canvas scalars are read.
  uint4 buf[DEPTH][NB * LPS];
#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d) load_batch<kBf16, NB>(buf[d], rsrc, byte_of(b_lo + d));

  // pieces of the supergroup each pair cuts, and the pair's arrival counts
  __shared__ float s_piece_ref[4][2][kWave];
  __shared__ float s_piece_sb[4][2][kWave];
  __shared__ uint32_t s_pair_arrivals[4];
  if (tid < 4) s_pair_arrivals[tid] = 0;
  __syncthreads();

  if (a.active != nullptr && !active_flag(a.active, canvas)) return;
  const float temp = a.temperature[canvas];
  const int32_t step = a.steps != nullptr ? a.steps[canvas] : a.step;
  const float c = kLog2e / temp;
  const uint64_t seed = a.seeds[canvas];
  const uint32_t k0 = static_cast<uint32_t>(seed);
  const uint32_t k1 = static_cast<uint32_t>(seed >> 32);

  LaneState st;
  auto consider = [&](float score, int32_t j) {
    if (score > st.best || (score == st.best && j < st.bestj)) {
      st.best = score;
      st.bestj = j;
    }
  };
  auto block_score = [&](int32_t j, float ref, float sb) {
    const Words4 rw = philox4x32_10(static_cast<uint32_t>(j), static_cast<uint32_t>(pos),
                                    static_cast<uint32_t>(step), kTagBlock, k0, k1);
    return ref + __log2f(sb) + kLog2e * gumbel(rw.w[0]);
  };
  // A block (this lane's slot across the 64 stripes of a supergroup) ends:
  // its score is its log-sum-exp plus its Gumbel, and its sums join the row's.
  // For the supergroup the pair cuts, this wave's piece goes to LDS instead;
  // the wave of the pair that closes its piece second combines both pieces.
  auto close_block = [&](int32_t b) {
    const int32_t sg = sg_of(b);
    const int32_t j = sg * kSlots + lane;
    if (sg == sg_cut) {
      s_piece_ref[pair][second][lane] = st.sb > 0.f ? st.ref : kNegInf;
      s_piece_sb[pair][second][lane] = st.sb;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      uint32_t prev = 0;
      if (lane == 0) prev = __hip_atomic_fetch_add(&s_pair_arrivals[pair], 1u, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_WORKGROUP);
      if (__builtin_amdgcn_readfirstlane(prev) == 1) {
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        const float r0 = s_piece_ref[pair][0][lane], r1 = s_piece_ref[pair][1][lane];
        const float q0 = s_piece_sb[pair][0][lane], q1 = s_piece_sb[pair][1][lane];
        const float rm = fmaxf(r0, r1);
        if (rm != kNegInf) {
          const float sum = (r0 == kNegInf ? 0.f : q0 * __builtin_amdgcn_exp2f(r0 - rm)) +
                            (r1 == kNegInf ? 0.f : q1 * __builtin_amdgcn_exp2f(r1 - rm));
          consider(block_score(j, rm, sum), j);
        }
      }
    } else if (st.sb > 0.f) {
      consider(block_score(j, st.ref, st.sb), j);
    }
    st.s += static_cast<double>(st.sb);
    st.w += static_cast<double>(st.wb);
    st.sb = 0.f;
    st.wb = 0.f;
  };

  // DEPTH divides a supergroup's batch count, so blocks end only after the
  // last batch of a ring turn.
  for (int32_t b = b_lo; b < n_fast; b += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      load_batch<kBf16, NB>(buf[(d + DEPTH - 1) % DEPTH], rsrc, byte_of(b + d + DEPTH - 1));
      if (b + d < n_fast)  // the loop has one exit, so load counters stay exact
        fast_batch<kBf16, NB>(buf[d], first_id(b + d), first_id(b + d) + lane * kSlotIds, vocab, c, st);
    }
    if ((b + DEPTH) % kBatchesPerSg == 0 && b + DEPTH <= n_fast) close_block(b);
  }
  if (n_fast < n) {
    // the batch that crosses V: loaded again here (ids past V read as zero and
    // are masked) and reduced on the slow path
    uint4 tb[NB * LPS];
    const int64_t bfirst = first_id(n - 1);
    load_batch<kBf16, NB>(tb, rsrc, static_cast<uint32_t>(bfirst) * kEB + lane_bytes);
    float z[NB * kSlotIds];
    unpack_batch<kBf16, NB>(tb, z);
    float bm = kNegInf;
#pragma unroll
    for (int q = 0; q < NB; ++q)
#pragma unroll
      for (int e = 0; e < kSlotIds; ++e)
        if (bfirst + lane * kSlotIds + q * kStripeIds + e < vocab) bm = fmaxf(bm, z[q * 8 + e]);
    if (bm > st.m) {
      st.m = bm;
      st.search = static_cast<int32_t>(bfirst);
    }
    slow_batch<kBf16, NB>(tb, bfirst + lane * kSlotIds, vocab, c, true, st);
  }
  if (n > b_lo && (n % kBatchesPerSg != 0 || n_fast < n)) close_block(n - 1);

  const RowPartial wp = wave_finish<kBf16, NB>(st, rsrc, vocab, temp, pos, step, k0, k1, lane);
  if (lane == 0) s_part[wave] = wp;
  __syncthreads();
  if (wave != 0) return;
  RowPartial p = merge_waves(s_part, lane);
  if (lane != 0) return;

  if (a.nsplit > 1) {
    // the last workgroup of the row (atomic ticket, release/acquire at agent
    // scope) merges every split's partial
    a.partials[static_cast<int64_t>(r) * a.nsplit + split] = p;
    __threadfence();
    const uint32_t prev = __hip_atomic_fetch_add(&a.tickets[r], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (prev != static_cast<uint32_t>(a.nsplit - 1)) return;
    __hip_atomic_store(&a.tickets[r], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __threadfence();
    const RowPartial* parts = a.partials + static_cast<int64_t>(r) * a.nsplit;
    p = parts[0];
    for (int sidx = 1; sidx < a.nsplit; ++sidx) merge_partial(p, parts[sidx]);
  }
  row_output(a, r, p);
}

}  // namespace

int32_t choose_nsplit(int32_t rows, int32_t vocab) {
  const int32_t nsg = (vocab + kSgIds - 1) / kSgIds;
  // aim for >= 2048 waves in flight (256 CUs x 8), at most one split per
  // kWaves supergroups so that every wave owns at least one supergroup
  int32_t want = (2048 / kWaves + rows - 1) / rows;
  int32_t cap = nsg / kWaves;
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want > 8) want = 8;
  return want < 1 ? 1 : want;
}

hipError_t launch_canvas_stats(const StatsArgs& a, bool bf16, hipStream_t stream) {
  const dim3 grid(static_cast<unsigned>(a.rows) * static_cast<unsigned>(a.nsplit));
  const dim3 block(kStatsThreads);
  if (bf16)
    hipLaunchKernelGGL((canvas_stats_kernel<true, 2, 4>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((canvas_stats_kernel<false, 2, 4>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace dg
