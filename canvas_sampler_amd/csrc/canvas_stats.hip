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
//     a block is one 8-id slot across the 8 stripes of a 4096-id chunk; each
//     lane forms its block's log-sum-exp on the fly and adds the block's
//     Gumbel, and the sample is the id of the best block j* with the largest
//     z/T + element Gumbel.
//
// Layout and schedule (gfx950, wave64): rows are V-contiguous. A workgroup of
// eight waves handles a row (or one split of it); with more rows than
// compute units a persistent grid loops over the rows. The two waves of a
// SIMD share its chunks s + 4p unevenly, the younger wave taking a quarter
// (the SIMD's arbiter favours the older one), so the workgroup reads nearby
// 4096-id chunks at any moment. Each lane issues one 16-byte load per 512-id stripe (bf16; two for
// fp32); a batch is 4 stripes and a block 2 batches, and a register ring
// holds two blocks: one is reduced while the other is in flight. The loops
// take the blocks in pairs so that every path into them leaves the two
// slots' loads in the same order and a block waits for its own loads only.
// Loads are raw buffer loads on a per-row resource (hardware range check, no
// branches), marked non-temporal; the per-canvas inputs are scalar loads, so
// they never wait behind the stream. Per element the loop costs one convert,
// half a max, one fma, one v_exp_f32, one add and one fma; per block one
// wave-uniform test for the rare cases, one log2 and two ballots. The block
// Gumbels: in the one-row kernel each wave draws its own as it goes (one
// Philox call per draw group of four chunks, kept in one of two register
// sets, no barrier before the stream); in the row loop the workgroup draws those of a whole
// segment of 64 chunks into LDS beforehand (the first while the first loads
// are in flight, the next ones before the barrier that ends a segment or a
// row). When a block ends its logits are still in registers, so nothing is
// read twice: if the block beats the wave's best block, or a lane of it holds
// a new wave maximum, that lane parks the block's 64 logits in LDS, and after
// its stream the wave finds the first id of its maximum from the parked
// logits. In the row loop each wave then finds the first id of its maximum,
// draws the sample in its best block and reduces its sums, and the workgroup
// merges eight 40-byte partials. In the one-row kernel each wave only
// publishes its lane sums and wave-level results, and after the barrier three
// waves finish the row at once: wave 0 the sums and the entropy, wave 1 the
// sample (drawn once, in the row's best block), wave 2 the first id of the
// maximum. The last wave to end its stream so reduces, searches and draws
// nothing before the barrier (measured at 256 x 262144 bf16, each change
// against the one before in one process: moving the draw off it 26.4 -> 25.9
// us, then the search and the sums 26.6 -> 26.1 us). A row split over
// several workgroups (for very short batches) writes one partial per split,
// its fields by those three waves.
//
// partials_merge_kernel merges, one wave per row and in a fixed order, the
// partials of split rows and the per-tile partials that the LM-head
// product's statistics epilogue writes. It runs as the next kernel on the
// stream: the kernel boundary orders the partials' stores before its loads,
// so no atomic ticket or agent-scope fence is needed (those cost about 24 us
// per launch at two splits per row).
#include <type_traits>

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

// Per-lane running state of the sums. The current block's sums stay in fp32
// (64 ids per lane, each term below 2^8 relative to ref) and are folded into
// the fp64 row sums when the block ends.
struct LaneState {
  double s = 0.0;        // sum 2^t over finished blocks, relative to ref
  double w = 0.0;        // sum t*2^t over finished blocks, relative to ref
  float sb = 0.f;        // current block's sum 2^t, relative to ref
  float wb = 0.f;        // current block's sum t*2^t, relative to ref
  float ref = kNegInf;   // reference, <= max z*c seen so far
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

// Reduces the batch that crosses V (ids past V masked) and returns its
// maximum raw logit below V.
template <bool kBf16, int NB>
__device__ __forceinline__ float tail_batch(const uint4 (&buf)[NB * Geometry<kBf16>::kLoadsPerStripe],
                                            int64_t id0, int32_t vocab, float c, LaneState& st) {
  float z[NB * kSlotIds];
  unpack_batch<kBf16, NB>(buf, z);
  float bm = kNegInf;
#pragma unroll
  for (int q = 0; q < NB; ++q)
#pragma unroll
    for (int e = 0; e < kSlotIds; ++e)
      if (id0 + q * kStripeIds + e < vocab) bm = fmaxf(bm, z[q * 8 + e]);
  slow_batch<kBf16, NB>(buf, id0, vocab, c, true, st);
  return bm;
}

// Logit e (0..7) of stripe s of a batch, as loaded.
template <bool kBf16, int NB>
__device__ __forceinline__ float batch_logit(const uint4 (&buf)[NB * Geometry<kBf16>::kLoadsPerStripe], int s,
                                             int e) {
  if constexpr (kBf16) {
    const uint4 q = buf[s];
    const uint32_t w = (e >> 1) == 0 ? q.x : (e >> 1) == 1 ? q.y : (e >> 1) == 2 ? q.z : q.w;
    return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
  } else {
    const uint4 q = buf[2 * s + (e >> 2)];
    const uint32_t w = (e & 3) == 0 ? q.x : (e & 3) == 1 ? q.y : (e & 3) == 2 ? q.z : q.w;
    return __uint_as_float(w);
  }
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

// Writes a row's outputs from its merged partial: H = ln 2 (log2 S - W/S).
__device__ __forceinline__ void row_output(const StatsArgs& a, int32_t r, const RowPartial& p, bool with_sample = true) {
  const double h = kLn2 * (log2(p.s) - p.w / p.s);
  const float hf = static_cast<float>(h);
  a.entropy[r] = hf > 0.0f ? hf : 0.0f;
  a.argmax[r] = p.argmax;
  if (with_sample) a.sample[r] = p.sample;
}

// Merges the eight wave partials across lanes 0..7 of wave 0 (lane l starts
// from partial l mod 8; three butterfly steps within each group of 8 lanes);
// lane 0 returns the merge of all eight. The argmax and the best block travel
// as 64-bit keys (a maximum decides both the value and the lowest-id tie
// break), the sample with its block; the entropy sums are rescaled once to the
// largest reference and then added.
__device__ __forceinline__ RowPartial merge_waves(const RowPartial* s_part, int lane) {
  const RowPartial q = s_part[lane & (kWaves - 1)];
  uint64_t km = argmax_key(q.m, q.argmax);
  uint64_t kb = argmax_key(q.best, q.bestj);
  int32_t sample = q.sample;
  float r = q.ref;
#define DG_MERGE_STEP(J)                                                               \
  {                                                                                    \
    km = max_u64(km, lane_xor64<J>(km));                                               \
    const uint64_t ob = lane_xor64<J>(kb);                                             \
    const int32_t os = static_cast<int32_t>(lane_xor<J>(static_cast<uint32_t>(sample))); \
    const bool take = ob > kb;                                                         \
    kb = take ? ob : kb;                                                               \
    sample = take ? os : sample;                                                       \
    r = max_raw(r, f32_of(lane_xor<J>(u32_of(r))));                                    \
  }
  DG_MERGE_STEP(4) DG_MERGE_STEP(2) DG_MERGE_STEP(1)
#undef DG_MERGE_STEP
  double s = 0.0, w = 0.0;
  if (q.ref != kNegInf) {
    const double d = static_cast<double>(q.ref) - static_cast<double>(r);
    const double f = scale_of(d);
    s = f * q.s;
    w = f * (q.w + d * q.s);
  }
#define DG_SUM_STEP(J)                                                                                        \
  s += __longlong_as_double(static_cast<long long>(lane_xor64<J>(static_cast<uint64_t>(__double_as_longlong(s))))); \
  w += __longlong_as_double(static_cast<long long>(lane_xor64<J>(static_cast<uint64_t>(__double_as_longlong(w)))));
  DG_SUM_STEP(4) DG_SUM_STEP(2) DG_SUM_STEP(1)
#undef DG_SUM_STEP
  RowPartial p;
  argmax_unkey(km, p.m, p.argmax);
  argmax_unkey(kb, p.best, p.bestj);
  p.sample = sample;
  p.ref = r;
  p.s = s;
  p.w = w;
  return p;
}

// Logit e (0..7) of stripe s of a block parked in LDS (the lane's 8 stripes,
// 16 bytes per stripe for bf16, 32 for fp32).
template <bool kBf16>
__device__ __forceinline__ float parked_logit(const uint4* blk, int s, int e) {
  if constexpr (kBf16) {
    const uint4 v4 = blk[s];
    const uint32_t w = (e >> 1) == 0 ? v4.x : (e >> 1) == 1 ? v4.y : (e >> 1) == 2 ? v4.z : v4.w;
    return __uint_as_float((e & 1) ? (w & 0xFFFF0000u) : (w << 16));
  } else {
    const uint4 v4 = blk[2 * s + (e >> 2)];
    return __uint_as_float((e & 3) == 0 ? v4.x : (e & 3) == 1 ? v4.y : (e & 3) == 2 ? v4.z : v4.w);
  }
}

// The wave's results so far (uniform across the wave): its maximum raw logit;
// the lowest id holding it when resolved (am_lane < 0), else the block (first
// id am_base) and the one lane holding it, whose logits wait in LDS; its best
// block score and block j, whose winning lane's logits wait in LDS.
struct WaveResult {
  float wm = kNegInf;
  int32_t wam = 0x7FFFFFFF;
  int64_t am_base = 0;
  int32_t am_lane = -1;
  float wbest = kNegInf;
  int32_t wbestj = 0x7FFFFFFF;
  int64_t best_base = 0;
};

// A wave's results as it ends its stream, published for the row's finish
// (one-row kernel): its maximum with its first id when already known
// (exact ties between lanes) or the lane whose parked block holds it, and
// its best block.
struct WaveEnd {
  float m;
  int32_t wam;
  int32_t am_lane;
  int64_t am_base;
  float best;
  int32_t bestj;
};

// Per-row constants of a pass.
struct RowConsts {
  int32_t pos;      // canvas position (counter word 1)
  int32_t step;     // counter word 2
  uint32_t k0, k1;  // Philox key: the canvas seed
  float c;          // log2(e) / T
  float inv_t;      // 1 / T: z/T as z * (1/T), within an ulp of the quotient
};

// Splits of a row start at multiples of 32 chunks, where the groups of four
// block draws that share a Philox call start (see fill_gumbels).
constexpr int32_t kDrawGroupChunks = 32;

// Blocks in flight per wave (the register ring's depth). Measured at 256 x
// 262144 (one-row kernel) and 16 x 256 x 262144 (row loop): bf16 rows 27.0
// us with two blocks against 28.0 with one; fp32 rows 50.0 us with one
// against 51.3 with two; the bf16 row loop 356 us with two against 384 with
// one.
template <bool kBf16>
constexpr int kRowRing = kBf16 ? 2 : 1;
constexpr int kRowsRing = 2;

// A segment: 64 consecutive chunks of a row (4096 blocks; the whole row at
// V = 262144), whose block Gumbels sit in LDS while its blocks are closed.
constexpr int32_t kSegChunks = 64;
constexpr int32_t kSegBlocks = kSegChunks * kSlots;


// The block Gumbels of the chunks [cb, ce) of the segment starting at chunk
// seg0, in log2 units: g2[(c - seg0) * 64 + slot] = log2(e) * G_j for block
// j = 64 c + slot. One Philox call serves the four blocks whose numbers differ
// only in bits 9-10 of j (chunks c0, c0 + 8, c0 + 16, c0 + 24 with bits 3-4 of
// c0 clear, inside an aligned group of 32 chunks): counter word 0 is j with
// those bits cleared and block j takes word (j >> 9) & 3. The workgroup's
// threads share the segment's 1024 calls.
__device__ __forceinline__ void fill_gumbels(float* g2, int32_t seg0, int32_t cb, int32_t ce, const RowConsts& rc,
                                             int tid) {
  for (int32_t i = tid; i < kSegBlocks / 4; i += kStatsThreads) {
    const int32_t c0 = seg0 + 32 * (i >> 9) + ((i >> 6) & 7);
    const int32_t slot = i & (kSlots - 1);
    if (c0 + 24 < cb || c0 >= ce) continue;
    const Words4 w = philox4x32_10(static_cast<uint32_t>(c0 * kSlots + slot), static_cast<uint32_t>(rc.pos),
                                   static_cast<uint32_t>(rc.step), kTagBlock, rc.k0, rc.k1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int32_t c = c0 + 8 * q;
      if (c >= cb && c < ce) g2[(c - seg0) * kSlots + slot] = kLog2e * gumbel(w.w[q]);
    }
  }
}

// The one-row kernel's chunk shares. The SIMD that runs waves s and s + 4
// owns the chunks s + 4p of every 64-chunk stretch (p < 16). Its arbiter
// favours the older wave (s): with equal shares (the younger wave on the odd
// p) the older waves end their streams at about 14 us of a 21 us pass and
// the younger ones stream the rest alone. So the younger wave takes only the
// positions in kYoungPositions, the older wave the others, each in increasing
// order. Measured at 256 x 262144 bf16 (statistics pass alone, the same run):
// 4 of 16 (the draw group of chunks s + 4 + 8q) 25.4-26.0 us against
// 25.9-26.6 us for equal shares; 5, 6 or a spread 5 of 16 were slower than 4.
// fp32 rows (256 x 262144): 46.4-46.7 us against 46.8-47.1.
constexpr uint32_t kYoungPositions = (1u << 1) | (1u << 3) | (1u << 5) | (1u << 7);

// The positions p of a 16-bit mask in increasing order, 4 bits each.
constexpr uint64_t packed_positions(uint32_t mask) {
  uint64_t r = 0;
  int n = 0;
  for (int p = 0; p < 16; ++p)
    if ((mask >> p) & 1u) r |= static_cast<uint64_t>(p) << (4 * n++);
  return r;
}

struct ChunkShare {
  int32_t c_begin;
  int sim;        // the SIMD's chunk residue s (wave & 3)
  uint32_t mask;  // the wave's positions in a stretch
  uint64_t pos;   // the same, packed
  int per;        // how many
  __device__ __forceinline__ ChunkShare(int32_t cb, int wave) : c_begin(cb), sim(wave & 3) {
    mask = wave >= 4 ? kYoungPositions : (~kYoungPositions & 0xFFFFu);
    pos = wave >= 4 ? packed_positions(kYoungPositions) : packed_positions(~kYoungPositions & 0xFFFFu);
    per = __builtin_popcount(mask);
  }
  // the chunk of the wave's block i
  __device__ __forceinline__ int32_t chunk(int32_t i) const {
    const int32_t k = i / per, n = i - k * per;
    return c_begin + 64 * k + sim + 4 * static_cast<int32_t>((pos >> (4 * n)) & 15u);
  }
  // the wave's blocks in chunks [c_begin, c_end)
  __device__ __forceinline__ int32_t count(int32_t c_end) const {
    const int32_t n = c_end - c_begin, full = n >> 6, rem = n & 63;
    const int32_t P = rem > sim ? (rem - sim + 3) >> 2 : 0;   // positions of the last, partial stretch
    return per * full + __builtin_popcount(mask & ((1u << P) - 1u));
  }
};

// The block Gumbels of a wave under ChunkShare: one Philox call per draw group
// (chunks c0 + 8q, c0 with bits 3-4 clear; c_begin is a multiple of 32), kept
// in one of two register sets; a wave's increasing chunks interleave at most
// two groups (the older wave's second half takes both groups of its residue),
// so no group is drawn twice.
struct ShareGumbels {
  int32_t ga = -1, gb = -1;   // the group in each set
  bool last_b = true;         // set b served the last block
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  float b0 = 0.f, b1 = 0.f, b2 = 0.f, b3 = 0.f;
  __device__ __forceinline__ float take(int32_t chunk, int lane, const RowConsts& rc) {
    const int32_t c0 = chunk & ~0x18;
    const int q = (chunk >> 3) & 3;
    bool use_a = c0 == ga;
    if (!use_a && c0 != gb) {
      const Words4 w = philox4x32_10(static_cast<uint32_t>(c0 * kSlots + lane), static_cast<uint32_t>(rc.pos),
                                     static_cast<uint32_t>(rc.step), kTagBlock, rc.k0, rc.k1);
      const float v0 = kLog2e * gumbel(w.w[0]), v1 = kLog2e * gumbel(w.w[1]);
      const float v2 = kLog2e * gumbel(w.w[2]), v3 = kLog2e * gumbel(w.w[3]);
      // the set not used last takes the group; selects, not a branch (a
      // branch lets the compiler turn the two sets into an indexed array in
      // scratch memory)
      use_a = last_b;
      a0 = use_a ? v0 : a0;
      a1 = use_a ? v1 : a1;
      a2 = use_a ? v2 : a2;
      a3 = use_a ? v3 : a3;
      b0 = use_a ? b0 : v0;
      b1 = use_a ? b1 : v1;
      b2 = use_a ? b2 : v2;
      b3 = use_a ? b3 : v3;
      ga = use_a ? c0 : ga;
      gb = use_a ? gb : c0;
    }
    last_b = !use_a;
    const float x0 = use_a ? a0 : b0, x1 = use_a ? a1 : b1;
    const float x2 = use_a ? a2 : b2, x3 = use_a ? a3 : b3;
    return q == 0 ? x0 : q == 1 ? x1 : q == 2 ? x2 : x3;
  }
};

template <bool kBf16, int NB, int R = 2>
using Ring = uint4[R][kChunkStripes / NB][NB * Geometry<kBf16>::kLoadsPerStripe];

// Block j (first id base, its 64 logits per lane in ring slot H) ends; bmax
// is the lane's maximum over them below V and g2 its Gumbel in log2 units.
template <bool kBf16, int NB, int H, int R>
__device__ __forceinline__ void close_block(const Ring<kBf16, NB, R>& buf, int64_t base, int32_t j, float bmax,
                                            float g2, LaneState& st, WaveResult& wr, uint4* park_best,
                                            uint4* park_max, int lane) {
  constexpr int LPS = Geometry<kBf16>::kLoadsPerStripe;
  // ---- argmax: the wave maximum rises. Blocks come in increasing id order,
  // so an equal later maximum never replaces an earlier one. With one holding
  // lane, that lane parks its logits and the first id is found after the pass;
  // with several (exact ties), the first id is found now. A holding lane's
  // first match lies below V: its ids increase with (stripe, e) and an id
  // below V holds the maximum.
  if (__builtin_amdgcn_ballot_w64(bmax > wr.wm) != 0) {
    const float m2 = wave_max(bmax);
    const uint64_t holders = __builtin_amdgcn_ballot_w64(bmax == m2);
    wr.wm = m2;
    if (__builtin_popcountll(holders) == 1) {
      wr.am_lane = static_cast<int32_t>(__builtin_ctzll(holders));
      wr.am_base = base;
      if (lane == wr.am_lane) {
#pragma unroll
        for (int q = 0; q < kChunkStripes * LPS; ++q) park_max[q] = buf[H][q / (NB * LPS)][q % (NB * LPS)];
      }
    } else {
      int32_t cand = 0x7FFFFFFF;
      if (bmax == m2) {
        int kf = 0;
#pragma unroll
        for (int k = kChunkStripes * kSlotIds - 1; k >= 0; --k) {
          const int s = k >> 3;
          kf = batch_logit<kBf16, NB>(buf[H][s / NB], s % NB, k & 7) == m2 ? k : kf;
        }
        cand = static_cast<int32_t>(base + (kf >> 3) * kStripeIds + lane * kSlotIds + (kf & 7));
      }
      wr.wam = wave_min_int(cand);
      wr.am_lane = -1;
    }
  }

  // ---- its score is its log-sum-exp plus its Gumbel
  float score = kNegInf;
  if (st.sb > 0.f) score = st.ref + __log2f(st.sb) + g2;
  st.s += static_cast<double>(st.sb);
  st.w += static_cast<double>(st.wb);
  st.sb = 0.f;
  st.wb = 0.f;

  // ---- a new best block of the wave (blocks in increasing order, so an equal
  // later score never replaces an earlier one): its winning lane parks the
  // block's logits; the sample is drawn in it after the pass.
  if (__builtin_amdgcn_ballot_w64(score > wr.wbest) != 0) {
    float sc = score;
    int32_t jj = j;
    wave_argmax(sc, jj);
    wr.wbest = sc;
    wr.wbestj = jj;
    wr.best_base = base;
    if (lane == (jj & (kSlots - 1))) {
#pragma unroll
      for (int q = 0; q < kChunkStripes * LPS; ++q) park_best[q] = buf[H][q / (NB * LPS)][q % (NB * LPS)];
    }
  }
}

// The in-block draw of the two-level sample: the Gumbel-max over the 64 ids
// of block j (first id base) parked in `park`, lane k taking logit e = k & 7
// of stripe k >> 3 (its ids increase with k). Every lane returns the id.
template <bool kBf16>
__device__ __forceinline__ int32_t draw_in_block(int64_t base, int32_t j, int32_t vocab, const RowConsts& rc,
                                                 const uint4* park, int lane) {
  const int sq = lane >> 3, e = lane & 7;
  const int wl = j & (kSlots - 1);
  const int64_t id = base + sq * kStripeIds + wl * kSlotIds + e;
  const Words4 g = philox4x32_10(static_cast<uint32_t>(id >> 2), static_cast<uint32_t>(rc.pos),
                                 static_cast<uint32_t>(rc.step), kTagElem, rc.k0, rc.k1);
  const uint32_t gw = (id & 3) == 0 ? g.w[0] : (id & 3) == 1 ? g.w[1] : (id & 3) == 2 ? g.w[2] : g.w[3];
  float s2 = id < vocab ? parked_logit<kBf16>(park, sq, e) * rc.inv_t + gumbel(gw) : kNegInf;
  int32_t id2 = static_cast<int32_t>(id);
  wave_argmax(s2, id2);
  return id2;
}

// The wave's partial once its blocks are done (row loop): the parked blocks
// give the first id of its maximum and the sample inside its best block; the
// sums are rescaled to the wave's largest reference. Every lane returns it.
template <bool kBf16>
__device__ __forceinline__ RowPartial wave_partial(const LaneState& st, const WaveResult& wr, int32_t vocab,
                                                   const RowConsts& rc, const uint4* park_best,
                                                   const uint4* park_max, int lane) {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  RowPartial p;
  const int sq = lane >> 3, e = lane & 7;
  p.argmax = wr.wam;
  if (wr.am_lane >= 0) {
    const int64_t id = wr.am_base + sq * kStripeIds + wr.am_lane * kSlotIds + e;
    const bool hit = id < vocab && parked_logit<kBf16>(park_max, sq, e) == wr.wm;
    const uint64_t hits = __builtin_amdgcn_ballot_w64(hit);  // never empty: the lane holds wm below V
    if (hits != 0) {
      const int k = static_cast<int>(__builtin_ctzll(hits));
      p.argmax = static_cast<int32_t>(wr.am_base + (k >> 3) * kStripeIds + wr.am_lane * kSlotIds + (k & 7));
    }
  }
  p.sample = 0x7FFFFFFF;
  if (wr.wbestj != 0x7FFFFFFF) p.sample = draw_in_block<kBf16>(wr.best_base, wr.wbestj, vocab, rc, park_best, lane);
  const float rr = wave_max(st.ref);
  double s = 0.0, w = 0.0;
  if (st.ref != kNegInf) {
    const double d = static_cast<double>(st.ref) - static_cast<double>(rr);
    const double f = scale_of(d);
    s = f * st.s;
    w = f * (st.w + d * st.s);
  }
  p.s = wave_sum(s);
  p.w = wave_sum(w);
  p.ref = rr;
  p.m = wr.wm;
  p.best = wr.wbest;
  p.bestj = wr.wbestj;
  return p;
}

// The sample of the best block over the eight waves' partials (the block
// merge_waves picks: largest score, lowest block among equal ones), drawn in
// the block its wave parked; 0x7FFFFFFF when no block has a score. Every
// lane returns it.
template <bool kBf16>
__device__ __forceinline__ int32_t draw_best(const WaveEnd* s_we, const uint4 (*park)[kChunkStripes * Geometry<kBf16>::kLoadsPerStripe],
                                             int32_t vocab, const RowConsts& rc, int lane) {
  const WaveEnd& q = s_we[lane & (kWaves - 1)];
  uint64_t kb = argmax_key(q.best, q.bestj);
  uint32_t wv = static_cast<uint32_t>(lane & (kWaves - 1));
#define DG_BEST_STEP(J)                  \
  {                                      \
    const uint64_t ob = lane_xor64<J>(kb); \
    const uint32_t ow = lane_xor<J>(wv);   \
    const bool take = ob > kb;           \
    kb = take ? ob : kb;                 \
    wv = take ? ow : wv;                 \
  }
  DG_BEST_STEP(4) DG_BEST_STEP(2) DG_BEST_STEP(1)
#undef DG_BEST_STEP
  const int w = __builtin_amdgcn_readfirstlane(static_cast<int>(wv));
  const int32_t j = __builtin_amdgcn_readfirstlane(s_we[w].bestj);
  if (j == 0x7FFFFFFF) return 0x7FFFFFFF;
  return draw_in_block<kBf16>(static_cast<int64_t>(j / kSlots) * kChunkIds, j, vocab, rc, park[w], lane);
}

// The row's maximum and the first id holding it, over the eight waves'
// published results (wave w's candidates in lanes 8 w .. 8 w + 7, lane 8 w + k
// searching stripe k of the block wave w parked); every lane returns them.
template <bool kBf16>
__device__ __forceinline__ void row_argmax(const WaveEnd* s_we,
                                           const uint4 (*park)[kChunkStripes * Geometry<kBf16>::kLoadsPerStripe],
                                           int32_t vocab, int lane, float& m, int32_t& am) {
  const int w = lane >> 3, sq = lane & 7;
  const WaveEnd& q = s_we[w];
  int32_t id = q.wam;
  if (q.am_lane >= 0) {
    id = 0x7FFFFFFF;
    const int64_t id0 = q.am_base + sq * kStripeIds + q.am_lane * kSlotIds;
#pragma unroll
    for (int e = 7; e >= 0; --e)
      id = id0 + e < vocab && parked_logit<kBf16>(park[w], sq, e) == q.m ? static_cast<int32_t>(id0 + e) : id;
  }
  id = min(id, static_cast<int32_t>(lane_xor<4>(static_cast<uint32_t>(id))));
  id = min(id, static_cast<int32_t>(lane_xor<2>(static_cast<uint32_t>(id))));
  id = min(id, static_cast<int32_t>(lane_xor<1>(static_cast<uint32_t>(id))));
  if (id == 0x7FFFFFFF) id = q.wam;  // (the holding lane's block always holds it below V)
  uint64_t k = argmax_key(q.m, id);
  k = max_u64(k, lane_xor64<8>(k));
  k = max_u64(k, lane_xor64<16>(k));
  k = max_u64(k, lane_xor64<32>(k));
  argmax_unkey(k, m, am);
}

// The row's sums over the 512 lanes' published sums, each rescaled once to
// the largest reference (lane l adds waves 0..7 of its column in order, then
// the wave sums the lanes); every lane returns them.
__device__ __forceinline__ void row_sums(const double (*s_ls)[kWave], const double (*s_lw)[kWave],
                                         const float (*s_lr)[kWave], int lane, double& s, double& w, float& ref) {
  float rl = kNegInf;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) rl = max_raw(rl, s_lr[v][lane]);
  const float r = wave_max(rl);
  double ls = 0.0, lw = 0.0;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) {
    const float q = s_lr[v][lane];
    if (q != kNegInf) {
      const double d = static_cast<double>(q) - static_cast<double>(r);
      const double f = scale_of(d);
      const double qs = s_ls[v][lane];
      ls += f * qs;
      lw += f * (s_lw[v][lane] + d * qs);
    }
  }
  s = wave_sum(ls);
  w = wave_sum(lw);
  ref = r;
}

// Reduces the batches of a full block in ring slot H into the lane state and
// returns the lane's maximum over them. The exponentials use the reference of
// the blocks before (it lags the running maximum), so each stripe is reduced
// as soon as its load lands instead of after a block-wide maximum; the block
// maximum is folded in afterwards. A lag of up to 2^64 cannot overflow fp32.
// One wave-uniform test per block catches the rare block that needs more: a
// lane's first finite logits, -inf logits (2^t = 0 but t*2^t = NaN), a
// maximum beyond the lag bound (the block is reduced again on the slow path,
// batch by batch) or above the reference's slack (the sums are rescaled).
template <bool kBf16, int NB, int H, int R>
__device__ __forceinline__ float reduce_block(const Ring<kBf16, NB, R>& buf, int64_t base, int32_t vocab, float c,
                                              LaneState& st, int lane) {
  constexpr float kMaxLag = 64.0f;
  float bs = 0.f, bw = 0.f, bmax = kNegInf;
#pragma unroll
  for (int t = 0; t < kChunkStripes / NB; ++t) {
    float s, w;
    bmax = max_raw(bmax, chunked_sums<kBf16, NB>(buf[H][t], c, st.ref, s, w));
    bs += s;
    bw += w;
    // one batch's temporaries at a time: the scheduler may not interleave
    // the batches (their exponentials would not fit the registers together)
    __builtin_amdgcn_sched_barrier(0);
  }
  const float bref = __fmul_rn(bmax, c);
  const bool bad = !(bw == bw) || !(bref <= st.ref + kMaxLag);  // NaN, fresh lane, or a big jump
  const bool lift = bref > st.ref + kRefSlack;
  if (__builtin_amdgcn_ballot_w64(bad || lift) != 0) {
    if (bad) {
#pragma unroll
      for (int t = 0; t < kChunkStripes / NB; ++t)
        slow_batch<kBf16, NB>(buf[H][t], base + t * NB * kStripeIds + lane * kSlotIds, vocab, c, false, st);
    } else {
      st.sb += bs;
      st.wb += bw;
    }
    if (bref > st.ref + kRefSlack) rebase(st, bref);
  } else {
    st.sb += bs;
    st.wb += bw;
  }
  return bmax;
}

template <bool kBf16, int NB, int H, int R>
__device__ __forceinline__ void load_block(Ring<kBf16, NB, R>& buf, __amdgpu_buffer_rsrc_t rsrc, uint32_t byte0,
                                           bool live) {
#pragma unroll
  for (int t = 0; t < kChunkStripes / NB; ++t)
    load_batch<kBf16, NB>(buf[H][t], rsrc,
                          live ? byte0 + static_cast<uint32_t>(t * NB * kStripeIds * Geometry<kBf16>::kElemBytes)
                               : kPastEnd);
}

template <bool kBf16>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const StatsArgs& a, int32_t r) {
  // The resource covers the row rounded up to 16 bytes (inside the row
  // stride): the range check works per dword, and a dword holding the last
  // bf16 id and one padding id must still be read. Ids past V are masked.
  constexpr int kEB = Geometry<kBf16>::kElemBytes;
  const char* row = static_cast<const char*>(a.logits) + static_cast<int64_t>(r) * a.row_stride * kEB;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(row), 0, ((a.vocab * kEB + 15) / 16) * 16, 0x00020000);
}

// A read-only input read through the constant address space: a scalar load,
// which waits on its own counter instead of behind the logits' vector loads
// in flight (the kernel never writes these arrays).
template <typename T>
__device__ __forceinline__ T read_only(const T* p, int32_t i) {
  return ((const __attribute__((address_space(4))) T*)p)[i];
}

__device__ __forceinline__ RowConsts row_consts(const StatsArgs& a, int32_t r) {
  const int32_t canvas = r / a.canvas_len;
  RowConsts rc;
  rc.pos = r % a.canvas_len;
  rc.step = a.steps != nullptr ? read_only(a.steps, canvas) : a.step;
  const float temp = read_only(a.temperature, canvas);
  rc.c = kLog2e / temp;
  rc.inv_t = 1.0f / temp;
  const uint64_t seed = read_only(a.seeds, canvas);
  rc.k0 = static_cast<uint32_t>(seed);
  rc.k1 = static_cast<uint32_t>(seed >> 32);
  return rc;
}

// One workgroup per row (or per split of a row). NB stripes per batch; the
// register ring holds RING blocks (one is reduced while the others are in
// flight). The waves share the chunks as ChunkShare says (a SIMD's chunks
// s + 4p, a quarter of them for its younger wave), and each draws the Gumbels
// of its own blocks as it goes (no barrier before the stream starts).
template <bool kBf16, int NB, int RING>
__global__ __launch_bounds__(kStatsThreads) void canvas_stats_kernel(StatsArgs a) {
  constexpr int LPS = Geometry<kBf16>::kLoadsPerStripe;
  constexpr uint32_t kEB = Geometry<kBf16>::kElemBytes;
  constexpr int kBB = kChunkStripes / NB;  // batches per block
  static_assert(kChunkStripes % NB == 0, "a block is a whole number of batches");
  // each wave's lane sums and wave-level results, published at its end
  __shared__ double s_ls[kWaves][kWave];   // lane sums of 2^t
  __shared__ double s_lw[kWaves][kWave];   // lane sums of t 2^t
  __shared__ float s_lr[kWaves][kWave];    // their references
  __shared__ WaveEnd s_we[kWaves];
  // per wave: the logits of its best block and of the block holding its
  // maximum (one lane's slot of a chunk each), kept for the end of the pass
  __shared__ __align__(16) uint4 s_blk[kWaves][kChunkStripes * LPS];
  __shared__ __align__(16) uint4 s_amx[kWaves][kChunkStripes * LPS];

  const int32_t r = static_cast<int32_t>(blockIdx.x) / a.nsplit;
  const int32_t split = static_cast<int32_t>(blockIdx.x) % a.nsplit;
  const int32_t canvas = r / a.canvas_len;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave index as a scalar, so the block loop below is uniform control flow
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int32_t vocab = a.vocab;
  const __amdgpu_buffer_rsrc_t rsrc = row_rsrc<kBf16>(a, r);
  const uint32_t lane_bytes = static_cast<uint32_t>(lane * kSlotIds) * kEB;

  // The split's chunks [c_begin, c_end), cut at multiples of 32 chunks. Each
  // wave takes its share (ChunkShare) in increasing order; only the row's
  // last chunk can be partial, and it is the last block of the wave that
  // holds it.
  const int32_t nchunk = (vocab + kChunkIds - 1) / kChunkIds;
  const int32_t ngroup = (nchunk + kDrawGroupChunks - 1) / kDrawGroupChunks;
  const int32_t c_begin = static_cast<int32_t>((static_cast<int64_t>(split) * ngroup) / a.nsplit) * kDrawGroupChunks;
  const int32_t c_end = min(static_cast<int32_t>((static_cast<int64_t>(split + 1) * ngroup) / a.nsplit) *
                            kDrawGroupChunks, nchunk);
  const ChunkShare cs(c_begin, wave);
  const int32_t nblk = cs.count(c_end);
  auto chunk_of = [&](int32_t i) { return cs.chunk(i); };
  auto base_of = [&](int32_t i) { return static_cast<int64_t>(chunk_of(i)) * kChunkIds; };
  // Block i's byte offset for this lane; batches wholly past V point beyond
  // the resource, where buffer loads return zero without touching memory, so
  // every load can be issued unconditionally.
  auto batch_byte = [&](int32_t i, int t) {
    const int64_t f = base_of(i) + t * NB * kStripeIds;
    return i < nblk && f < vocab ? static_cast<uint32_t>(f) * kEB + lane_bytes : kPastEnd;
  };
  // Blocks [0, nblk_full) lie wholly below V; the block holding V, if any, is
  // the wave's last and is reduced after the loop.
  const int32_t nblk_full =
      (nblk > 0 && base_of(nblk - 1) + kChunkIds > vocab) ? nblk - 1 : nblk;

  // The ring: its first blocks go out before the per-canvas scalars are read.
  Ring<kBf16, NB, RING> buf;
#pragma unroll
  for (int h = 0; h < RING; ++h)
#pragma unroll
    for (int t = 0; t < kBB; ++t) load_batch<kBf16, NB>(buf[h][t], rsrc, batch_byte(h, t));

  if (a.active != nullptr && !active_flag(a.active, canvas)) return;
  const RowConsts rc = row_consts(a, r);
  LaneState st;
  WaveResult wr;
  ShareGumbels gw;

  // Full blocks: reduce, close, and refill the ring slot with block i + RING.
  auto run_block = [&](auto slot, int32_t i) {
    constexpr int H = decltype(slot)::value;
    const float bmax = reduce_block<kBf16, NB, H>(buf, base_of(i), vocab, rc.c, st, lane);
    const float g2 = gw.take(chunk_of(i), lane, rc);
    close_block<kBf16, NB, H>(buf, base_of(i), chunk_of(i) * kSlots + lane, bmax, g2, st, wr, s_blk[wave],
                              s_amx[wave], lane);
#pragma unroll
    for (int t = 0; t < kBB; ++t) load_batch<kBf16, NB>(buf[H][t], rsrc, batch_byte(i + RING, t));
  };
  // block i waits in ring slot i % RING; the loop takes the slots in turn, so
  // that every way into it leaves their loads in the same order and each
  // block waits for its own loads only; a last odd block follows it
  int32_t i = 0;
  if constexpr (RING == 1) {
    for (; i < nblk_full; ++i) run_block(std::integral_constant<int, 0>{}, i);
  } else {
    for (; i + 1 < nblk_full; i += 2) {
      run_block(std::integral_constant<int, 0>{}, i);
      run_block(std::integral_constant<int, 1>{}, i + 1);
    }
    if (i < nblk_full) {
      run_block(std::integral_constant<int, 0>{}, i);
      ++i;
    }
  }
  if (nblk_full < nblk) {
    // the block holding V sits in ring slot i % RING (moved to slot 0);
    // batches below V are reduced with ids past V masked, the rest skipped
    if (RING > 1 && (i & 1)) {
#pragma unroll
      for (int t = 0; t < kBB; ++t)
#pragma unroll
        for (int q = 0; q < NB * LPS; ++q) buf[0][t][q] = buf[RING - 1][t][q];
    }
    float bmax = kNegInf;
#pragma unroll
    for (int t = 0; t < kBB; ++t) {
      const int64_t f = base_of(i) + t * NB * kStripeIds;
      if (f < vocab) bmax = fmaxf(bmax, tail_batch<kBf16, NB>(buf[0][t], f + lane * kSlotIds, vocab, rc.c, st));
    }
    const float g2 = gw.take(chunk_of(i), lane, rc);
    close_block<kBf16, NB, 0>(buf, base_of(i), chunk_of(i) * kSlots + lane, bmax, g2, st, wr, s_blk[wave],
                              s_amx[wave], lane);
  }

  // Each wave publishes its lane sums and wave-level results and leaves; the
  // row's finish is then split over three waves at once: wave 0 the sums and
  // the entropy, wave 1 the sample (drawn once, in the row's best block),
  // wave 2 the first id of the maximum. The last wave to end its stream so
  // does no reduction, search or draw before the barrier.
  s_ls[wave][lane] = st.s;
  s_lw[wave][lane] = st.w;
  s_lr[wave][lane] = st.ref;
  if (lane == 0) s_we[wave] = WaveEnd{wr.wm, wr.wam, wr.am_lane, wr.am_base, wr.wbest, wr.wbestj};
  __syncthreads();
  RowPartial* part = a.nsplit > 1 ? a.partials + static_cast<int64_t>(r) * a.nsplit + split : nullptr;
  if (wave == 0) {
    RowPartial p;
    row_sums(s_ls, s_lw, s_lr, lane, p.s, p.w, p.ref);
    if (lane != 0) return;
    if (part != nullptr) {
      // a split's partial, written by waves 0-2 field by field;
      // partials_merge_kernel, next on the stream, merges them
      part->s = p.s;
      part->w = p.w;
      part->ref = p.ref;
      return;
    }
    const double h = kLn2 * (log2(p.s) - p.w / p.s);
    const float hf = static_cast<float>(h);
    a.entropy[r] = hf > 0.0f ? hf : 0.0f;
  } else if (wave == 1) {
    const int32_t smp = draw_best<kBf16>(s_we, s_blk, vocab, rc, lane);
    if (lane != 0) return;
    if (part != nullptr) {
      int32_t bj = 0x7FFFFFFF;
      float bs = kNegInf;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const uint64_t cand = argmax_key(s_we[v].best, s_we[v].bestj);
        if (cand > argmax_key(bs, bj)) {
          bs = s_we[v].best;
          bj = s_we[v].bestj;
        }
      }
      part->best = bs;
      part->bestj = bj;
      part->sample = smp;
      return;
    }
    a.sample[r] = smp;
  } else if (wave == 2) {
    float m;
    int32_t am;
    row_argmax<kBf16>(s_we, s_amx, vocab, lane, m, am);
    if (lane != 0) return;
    if (part != nullptr) {
      part->m = m;
      part->argmax = am;
      return;
    }
    a.argmax[r] = am;
  }
}

// Row loop: a persistent grid of workgroups, workgroup b taking rows b,
// b + grid, ... (V a multiple of 4096, one workgroup per row, no active
// mask). Wave w streams chunks w, w + 8, ... of each row, and its blocks of
// all its rows form one sequence g = 0, 1, ...; the ring refills slot g % 2
// with block g + 2 even when that block belongs to the next row, so a row's
// finish and merge overlap the next row's loads. The block Gumbels of each
// segment of 64 chunks are drawn into one of two LDS tables by the waves that
// have finished the segment before, in the barrier that ends it.
template <bool kBf16, int NB, bool kSeg, bool kPairs, int RING>
__global__ __launch_bounds__(kStatsThreads) void canvas_stats_rows_kernel(StatsArgs a) {
  constexpr int LPS = Geometry<kBf16>::kLoadsPerStripe;
  constexpr uint32_t kEB = Geometry<kBf16>::kElemBytes;
  __shared__ RowPartial s_part[2][kWaves];  // by row parity
  __shared__ __align__(16) uint4 s_blk[kWaves][kChunkStripes * LPS];
  __shared__ __align__(16) uint4 s_amx[kWaves][kChunkStripes * LPS];
  __shared__ float s_g2[2][kSegBlocks];     // by segment parity

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int32_t vocab = a.vocab;
  const uint32_t lane_bytes = static_cast<uint32_t>(lane * kSlotIds) * kEB;
  const int32_t grid = static_cast<int32_t>(gridDim.x);
  const int32_t first_row = static_cast<int32_t>(blockIdx.x);
  const int32_t my_rows = (a.rows - first_row + grid - 1) / grid;  // >= 1
  const int32_t nchunk = vocab / kChunkIds;
  // the wave's chunks of a row as in the one-row kernel (ChunkShare); the
  // segments' Gumbel tables serve any share. Measured (same process, N(0,1)
  // bf16 rows of 262144): 16 canvases 340.7-340.9 us against 341.1-343.7 with
  // equal shares, 64 canvases 1.324-1.325 ms against 1.338-1.339.
  const ChunkShare cs(0, wave);
  auto blocks_below = [&](int32_t c) { return cs.count(c); };
  const int32_t nblk = blocks_below(nchunk);  // per row
  const int64_t total = static_cast<int64_t>(my_rows) * nblk;

  // Block g of the wave's sequence is block g % nblk (chunk cs.chunk(g % nblk))
  // of row first_row + (g / nblk) * grid; past the sequence, loads read nothing.
  Ring<kBf16, NB, RING> buf;
  auto fetch = [&](auto slot, int64_t g) {
    constexpr int H = decltype(slot)::value;
    int32_t r = first_row;
    uint32_t byte0 = 0;
    const bool live = g < total;
    if (live) {
      r = first_row + static_cast<int32_t>(g / nblk) * grid;
      byte0 = static_cast<uint32_t>(cs.chunk(static_cast<int32_t>(g % nblk))) * (kChunkIds * kEB) + lane_bytes;
    }
    load_block<kBf16, NB, H>(buf, row_rsrc<kBf16>(a, r), byte0, live);
  };
  fetch(std::integral_constant<int, 0>{}, 0);
  if constexpr (RING > 1) fetch(std::integral_constant<int, RING - 1>{}, 1);

  RowConsts rc = row_consts(a, first_row);
  fill_gumbels(s_g2[0], 0, 0, min(nchunk, kSegChunks), rc, tid);
  __syncthreads();
  int tp = 0;  // table in use
  int64_t g = 0;
  for (int32_t k = 0; k < my_rows; ++k) {
    const int32_t r = first_row + k * grid;
    LaneState st;
    WaveResult wr;
    const RowConsts rc_next = k + 1 < my_rows ? row_consts(a, r + grid) : rc;
    // block i of the row, block gi of the wave's sequence, in ring slot gi % 2
    auto run_block = [&](auto slot, int32_t i, int64_t gi, int32_t seg0) {
      constexpr int H = decltype(slot)::value;
      const int32_t chunk = cs.chunk(i);
      const float gv = s_g2[tp][(chunk - seg0) * kSlots + lane];
      const int64_t base = static_cast<int64_t>(chunk) * kChunkIds;
      const float bmax = reduce_block<kBf16, NB, H>(buf, base, vocab, rc.c, st, lane);
      close_block<kBf16, NB, H>(buf, base, chunk * kSlots + lane, bmax, gv, st, wr, s_blk[wave], s_amx[wave], lane);
      fetch(slot, gi + RING);
    };
    // the end of a segment: the next segment's Gumbels (this row's next, or
    // the next row's first) go into the other table, and at the row's end
    // the wave's partial into s_part, both published by the barrier
    auto end_segment = [&](int32_t seg_end) {
      const bool last_seg = seg_end >= nchunk;
      if (!last_seg)
        fill_gumbels(s_g2[tp ^ 1], seg_end, seg_end, min(nchunk, seg_end + kSegChunks), rc, tid);
      else if (k + 1 < my_rows)
        fill_gumbels(s_g2[tp ^ 1], 0, 0, min(nchunk, kSegChunks), rc_next, tid);
      if (last_seg) {
        const RowPartial wp = wave_partial<kBf16>(st, wr, vocab, rc, s_blk[wave], s_amx[wave], lane);
        if (lane == 0) s_part[k & 1][wave] = wp;
      }
      __syncthreads();
      tp ^= 1;
    };
    if constexpr (RING == 1) {
      // one block in flight per wave, always in the ring's only slot
      for (int32_t seg0 = 0; seg0 < nchunk; seg0 += kSegChunks) {
        const int32_t seg_end = min(nchunk, seg0 + kSegChunks);
        for (int32_t i = blocks_below(seg0); i < blocks_below(seg_end); ++i, ++g)
          run_block(std::integral_constant<int, 0>{}, i, g, seg0);
        end_segment(seg_end);
      }
    } else if constexpr (kPairs) {
      // one segment per row and an even number of blocks per wave (chunks a
      // multiple of 16): every row starts in slot 0, and a loop over pairs
      // keeps the two slots' loads in order, so that each block waits for
      // its own loads alone
      for (int32_t i = 0; i < nblk; i += 2, g += 2) {
        run_block(std::integral_constant<int, 0>{}, i, g, 0);
        run_block(std::integral_constant<int, RING - 1>{}, i + 1, g + 1, 0);
      }
      end_segment(nchunk);
    } else if constexpr (!kSeg) {
      // one segment per row (rows of up to 262144 ids)
      for (int32_t i = 0; i < nblk; ++i, ++g) {
        if ((g & 1) == 0)
          run_block(std::integral_constant<int, 0>{}, i, g, 0);
        else
          run_block(std::integral_constant<int, RING - 1>{}, i, g, 0);
      }
      end_segment(nchunk);
    } else {
      for (int32_t seg0 = 0; seg0 < nchunk; seg0 += kSegChunks) {
        const int32_t seg_end = min(nchunk, seg0 + kSegChunks);
        for (int32_t i = blocks_below(seg0); i < blocks_below(seg_end); ++i, ++g) {
          if ((g & 1) == 0)
            run_block(std::integral_constant<int, 0>{}, i, g, seg0);
          else
            run_block(std::integral_constant<int, RING - 1>{}, i, g, seg0);
        }
        end_segment(seg_end);
      }
    }
    // the merge of row k falls to wave k mod 8; the other waves go on. The
    // partials are double-buffered by row parity: row k + 2 writes them only
    // after the barrier of row k + 1, which the merging wave reaches after
    // its merge.
    if (wave == (k & (kWaves - 1))) {
      const RowPartial p = merge_waves(s_part[k & 1], lane);
      if (lane == 0) row_output(a, r, p);
    }
    rc = rc_next;
  }
}

// Merges the partials of the 64 lanes of a wave (lane l holds the merge of
// its share of a row's partials): a butterfly over the maxima and best-block
// keys, then the sums rescaled once to the largest reference and added.
// Every lane returns the result.
__device__ __forceinline__ RowPartial merge_lanes(const RowPartial& q) {
  uint64_t km = argmax_key(q.m, q.argmax);
  uint64_t kb = argmax_key(q.best, q.bestj);
  int32_t sample = q.sample;
  float r = q.ref;
#define DG_MERGE_STEP(J)                                                               \
  {                                                                                    \
    km = max_u64(km, lane_xor64<J>(km));                                               \
    const uint64_t ob = lane_xor64<J>(kb);                                             \
    const int32_t os = static_cast<int32_t>(lane_xor<J>(static_cast<uint32_t>(sample))); \
    const bool take = ob > kb;                                                         \
    kb = take ? ob : kb;                                                               \
    sample = take ? os : sample;                                                       \
    r = max_raw(r, f32_of(lane_xor<J>(u32_of(r))));                                    \
  }
  DG_MERGE_STEP(32) DG_MERGE_STEP(16) DG_MERGE_STEP(8) DG_MERGE_STEP(4) DG_MERGE_STEP(2) DG_MERGE_STEP(1)
#undef DG_MERGE_STEP
  double s = 0.0, w = 0.0;
  if (q.ref != kNegInf) {
    const double d = static_cast<double>(q.ref) - static_cast<double>(r);
    const double f = scale_of(d);
    s = f * q.s;
    w = f * (q.w + d * q.s);
  }
  RowPartial p;
  argmax_unkey(km, p.m, p.argmax);
  argmax_unkey(kb, p.best, p.bestj);
  p.sample = sample;
  p.ref = r;
  p.s = wave_sum(s);
  p.w = wave_sum(w);
  return p;
}

constexpr int kMergeThreads = 256;

// One wave per row: lane l merges the row's partials l, l + 64, ... in order,
// then the wave merges its lanes and lane 0 writes the row's outputs. Rows of
// inactive canvases are skipped (their outputs are not written).
__global__ __launch_bounds__(kMergeThreads) void partials_merge_kernel(StatsArgs a, const RowPartial* parts,
                                                                       int32_t nparts) {
  const int lane = threadIdx.x & (kWave - 1);
  const int32_t r = static_cast<int32_t>(blockIdx.x) * (kMergeThreads / kWave) +
                    __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  if (r >= a.rows) return;
  if (a.active != nullptr && !active_flag(a.active, r / a.canvas_len)) return;
  const RowPartial* row = parts + static_cast<int64_t>(r) * nparts;
  RowPartial p;
  p.s = 0.0;
  p.w = 0.0;
  p.ref = kNegInf;
  p.m = kNegInf;
  p.argmax = 0x7FFFFFFF;
  p.best = kNegInf;
  p.bestj = 0x7FFFFFFF;
  p.sample = 0x7FFFFFFF;
  for (int32_t t = lane; t < nparts; t += kWave) merge_partial(p, row[t]);
  p = merge_lanes(p);
  if (lane == 0) row_output(a, r, p);
}

}  // namespace

hipError_t launch_partials_merge(const StatsArgs& a, const RowPartial* partials, int32_t nparts,
                                 hipStream_t stream) {
  constexpr int kRowsPerBlock = kMergeThreads / kWave;
  const dim3 grid(static_cast<unsigned>((a.rows + kRowsPerBlock - 1) / kRowsPerBlock));
  hipLaunchKernelGGL(partials_merge_kernel, grid, dim3(kMergeThreads), 0, stream, a, partials, nparts);
  return hipGetLastError();
}

int32_t choose_nsplit(int32_t rows, int32_t vocab) {
  const int32_t nchunk = (vocab + kChunkIds - 1) / kChunkIds;
  // Split a row over two workgroups while the splits stay within the 256
  // CUs' one resident workgroup each: the splits' partials are merged by the
  // next kernel on the stream. Measured at V = 262144 bf16, statistics and
  // merge, one / two / four workgroups per row: L = 16 21.5 / 18.3 / 18.8 us,
  // L = 32 22.0 / 18.3 / 18.7 us, L = 64 22.2 / 18.7 / 19.4 us, L = 128
  // 22.5 / 21.3 / 33.2 us, L = 256 26.5 / 36.0 / 60.4 us. At most one split
  // per 32 chunks: splits start at multiples of 32 chunks, where the groups of
  // four block draws start.
  int32_t want = rows <= 128 ? 2 : 1;
  int32_t cap = nchunk / kDrawGroupChunks;
  if (cap < 1) cap = 1;
  return want > cap ? cap : want;
}

int32_t stats_row_grid(int32_t rows, int32_t vocab, int32_t nsplit, bool has_active, int32_t cu_count) {
  // the row loop needs whole chunks, one workgroup per row and every row to be
  // processed; it pays off once there are more rows than resident workgroups
  // (one per CU at this kernel's register use)
  if (nsplit != 1 || has_active || vocab % kChunkIds != 0 || cu_count < 1 || rows <= cu_count) return 0;
  return cu_count;
}

hipError_t launch_canvas_stats(const StatsArgs& a, bool bf16, hipStream_t stream) {
  const dim3 block(kStatsThreads);
  // rows of more than one segment (64 chunks, 262144 ids) take the kernels'
  // segment loops; shorter rows the plain ones
  const int32_t nchunk = (a.vocab + kChunkIds - 1) / kChunkIds;
  const bool seg = nchunk > kSegChunks;
  if (a.row_grid > 0) {
    const dim3 grid(static_cast<unsigned>(a.row_grid));
    const bool pairs = kRowsRing == 2 && !seg && nchunk % 16 == 0;
#define DG_ROWS(BF, SEG, PAIRS) \
  hipLaunchKernelGGL((canvas_stats_rows_kernel<BF, 4, SEG, PAIRS, kRowsRing>), grid, block, 0, stream, a)
    if (bf16) {
      if (pairs) DG_ROWS(true, false, true);
      else if (seg) DG_ROWS(true, true, false);
      else DG_ROWS(true, false, false);
    } else {
      if (pairs) DG_ROWS(false, false, true);
      else if (seg) DG_ROWS(false, true, false);
      else DG_ROWS(false, false, false);
    }
#undef DG_ROWS
  } else {
    const dim3 grid(static_cast<unsigned>(a.rows) * static_cast<unsigned>(a.nsplit));
    if (bf16)
      hipLaunchKernelGGL((canvas_stats_kernel<true, 4, kRowRing<true>>), grid, block, 0, stream, a);
    else
      hipLaunchKernelGGL((canvas_stats_kernel<false, 4, kRowRing<false>>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace dg

