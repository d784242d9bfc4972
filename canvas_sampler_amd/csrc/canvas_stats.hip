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
// four waves handles one split (a range of 32768-id supergroups) of one row;
// its waves take supergroups round-robin. Each lane issues one 16-byte load
// per 512-id stripe (bf16; two for fp32), so a wave's load covers 1 KiB (bf16)
// or 2 KiB (fp32) of consecutive memory; loads of the next batch of stripes
// are issued before the current batch is reduced (register double buffer).
// Per element the loop costs one convert, half a max, one fma, one v_exp_f32,
// one add and one fma; the per-block and per-batch work is amortised over 64
// ids per lane. When a row is split over several workgroups, each writes a
// 32-byte partial and the last one to finish (atomic ticket, release/acquire
// at agent scope) merges them and finishes the row.
#include "device_common.h"
#include "kernels.h"

namespace dg {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.69314718055994530942;
constexpr int kWaves = kStatsThreads / kWave;
constexpr float kNegInf = -__builtin_inff();

// Lets the running reference trail the true maximum by up to 8 (log2 units,
// a factor 256) before the sums are rescaled: 2^t <= 256 cannot overflow.
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

// Per-lane running state of the pass.
struct LaneState {
  double s = 0.0;        // sum 2^t relative to ref
  double w = 0.0;        // sum t*2^t relative to ref
  double sb = 0.0;       // current block's sum 2^t relative to ref
  float ref = kNegInf;   // reference, <= max z*c seen so far
  float m = kNegInf;     // max raw logit
  int32_t search = 0x7FFFFFFF;
  float best = kNegInf;  // best block score (log2 units)
  int32_t bestj = 0x7FFFFFFF;
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

template <bool kBf16, int NB>
__device__ __forceinline__ void process_batch(const uint4 (&buf)[NB * Geometry<kBf16>::kLoadsPerStripe],
                                              int64_t id0, int64_t batch_first_id, int32_t vocab,
                                              float c, LaneState& st) {
  float z[NB * kSlotIds];
  unpack_batch<kBf16, NB>(buf, z);
  if (batch_first_id + NB * kStripeIds > vocab) {
    // the batch holding id V-1: ids past V (read as zero) become -inf
#pragma unroll
    for (int s = 0; s < NB; ++s)
#pragma unroll
      for (int e = 0; e < kSlotIds; ++e)
        if (id0 + s * kStripeIds + e >= vocab) z[s * 8 + e] = kNegInf;
  }
  float bm = z[0];
#pragma unroll
  for (int k = 1; k < NB * kSlotIds; ++k) bm = fmaxf(bm, z[k]);
  // exact argmax bookkeeping: first batch that attains the lane's maximum
  if (bm > st.m) {
    st.m = bm;
    st.search = static_cast<int32_t>(batch_first_id >> 13);
  }
  const float bref = __fmul_rn(bm, c);
  if (bref > st.ref + kRefSlack) {
    if (st.ref != kNegInf) {
      const double d = static_cast<double>(st.ref) - static_cast<double>(bref);
      const double f = exp2(d);
      st.w = f * (st.w + d * st.s);
      st.s *= f;
      st.sb *= f;
    }
    st.ref = bref;
  }
  if (st.ref == kNegInf) return;  // nothing finite seen by this lane yet
  float bs, bw;
  batch_sums<NB * kSlotIds>(z, c, st.ref, bs, bw);
  st.s += static_cast<double>(bs);
  st.w += static_cast<double>(bw);
  st.sb += static_cast<double>(bs);
}

// Merges partial b into a (entropy sums, argmax, best block).
__device__ __forceinline__ void merge_partial(RowPartial& a, const RowPartial& b) {
  if (b.m > a.m || (b.m == a.m && b.search < a.search)) {
    a.m = b.m;
    a.search = b.search;
  }
  if (b.best > a.best || (b.best == a.best && b.bestj < a.bestj)) {
    a.best = b.best;
    a.bestj = b.bestj;
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
  const double fa = exp2(da), fb = exp2(db);
  a.w = fa * (a.w + da * a.s) + fb * (b.w + db * b.s);
  a.s = fa * a.s + fb * b.s;
  a.ref = r;
}

// Reduces the lane states of a wave into one partial (valid in every lane).
__device__ __forceinline__ RowPartial wave_partial(const LaneState& st) {
  RowPartial p;
  const float r = wave_max(st.ref);
  double s = 0.0, w = 0.0;
  if (st.ref != kNegInf) {
    const double d = static_cast<double>(st.ref) - static_cast<double>(r);
    const double f = exp2(d);
    s = f * st.s;
    w = f * (st.w + d * st.s);
  }
  p.s = wave_sum(s);
  p.w = wave_sum(w);
  p.ref = r;
  p.m = wave_max(st.m);
  p.search = wave_min_int(st.m == p.m ? st.search : 0x7FFFFFFF);
  float best = st.best;
  int bestj = st.bestj;
  wave_argmax(best, bestj);
  p.best = best;
  p.bestj = bestj;
  p.pad = 0;
  return p;
}

// Finishes a row from its merged partial: entropy, exact argmax (re-search of
// one 8192-id unit), and the in-block resample of block j*. Every thread of
// the workgroup takes part with unconditional buffer loads (ids past V read
// as zero and are excluded), so each phase costs one memory latency; thread 0
// writes the results.
template <bool kBf16>
__device__ void finish_row(const StatsArgs& a, __amdgpu_buffer_rsrc_t rsrc, int32_t r,
                           int32_t pos, float temp, uint32_t k0, uint32_t k1,
                           const RowPartial& p) {
  constexpr uint32_t kEB = Geometry<kBf16>::kElemBytes;
  constexpr int kChunksPerThread = kSearchIds / (kStatsThreads * kSlotIds);
  __shared__ int32_t s_min[kWaves];
  __shared__ float s_score[kWaves];
  __shared__ int32_t s_id[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int32_t vocab = a.vocab;

  // exact argmax: lowest id of the unit whose value equals the maximum
  int32_t cand = 0x7FFFFFFF;
  {
    const int64_t base = static_cast<int64_t>(p.search) * kSearchIds;
    float z[kChunksPerThread][kSlotIds];
#pragma unroll
    for (int i = 0; i < kChunksPerThread; ++i) {
      const int64_t id0 = base + static_cast<int64_t>(i * kStatsThreads + tid) * kSlotIds;
      const uint32_t off = id0 < vocab ? static_cast<uint32_t>(id0) * kEB : kPastEnd;
      if constexpr (kBf16) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, static_cast<int>(off), 0, 0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          z[i][2 * q] = __uint_as_float(v[q] << 16);
          z[i][2 * q + 1] = __uint_as_float(v[q] & 0xFFFF0000u);
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const auto v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, static_cast<int>(off + 16 * h), 0, 0);
#pragma unroll
          for (int q = 0; q < 4; ++q) z[i][4 * h + q] = __uint_as_float(v[q]);
        }
      }
    }
#pragma unroll
    for (int i = kChunksPerThread - 1; i >= 0; --i) {
      const int64_t id0 = base + static_cast<int64_t>(i * kStatsThreads + tid) * kSlotIds;
#pragma unroll
      for (int e = kSlotIds - 1; e >= 0; --e)
        if (id0 + e < vocab && z[i][e] == p.m) cand = static_cast<int32_t>(id0 + e);
    }
  }
  cand = wave_min_int(cand);

  // in-block resample: the 512 members of block j*, one per thread
  float best = kNegInf;
  int32_t best_id = 0x7FFFFFFF;
  {
    const int32_t j = p.bestj;
    const int64_t v = static_cast<int64_t>(j >> 6) * kSgIds + static_cast<int64_t>(tid >> 3) * kStripeIds +
                      (j & 63) * kSlotIds + (tid & 7);
    const uint32_t off = v < vocab ? static_cast<uint32_t>(v) * kEB : kPastEnd;
    float zv;
    if constexpr (kBf16) {
      const uint16_t bits = __builtin_amdgcn_raw_buffer_load_b16(rsrc, static_cast<int>(off), 0, 0);
      zv = __uint_as_float(static_cast<uint32_t>(bits) << 16);
    } else {
      zv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc, static_cast<int>(off), 0, 0));
    }
    const Words4 rw = philox4x32_10(static_cast<uint32_t>(v >> 2), static_cast<uint32_t>(pos),
                                    static_cast<uint32_t>(a.step), kTagElem, k0, k1);
    if (v < vocab) {
      best = zv / temp + gumbel(rw.w[v & 3]);
      best_id = static_cast<int32_t>(v);
    }
  }
  wave_argmax(best, best_id);
  if (lane == 0) {
    s_min[wave] = cand;
    s_score[wave] = best;
    s_id[wave] = best_id;
  }
  __syncthreads();
  if (tid == 0) {
    int32_t am = s_min[0];
    float bs = s_score[0];
    int32_t bid = s_id[0];
    for (int w = 1; w < kWaves; ++w) {
      am = min(am, s_min[w]);
      if (s_score[w] > bs || (s_score[w] == bs && s_id[w] < bid)) {
        bs = s_score[w];
        bid = s_id[w];
      }
    }
    const double h = kLn2 * (log2(p.s) - p.w / p.s);
    const float hf = static_cast<float>(h);
    a.entropy[r] = hf > 0.0f ? hf : 0.0f;
    a.argmax[r] = am;
    a.sample[r] = bid;
  }
}

template <bool kBf16, int NB>
__global__ __launch_bounds__(kStatsThreads) void canvas_stats_kernel(StatsArgs a) {
  constexpr int LPS = Geometry<kBf16>::kLoadsPerStripe;
  constexpr int kBatchesPerSg = kStripesPerSg / NB;
  __shared__ RowPartial s_part[kWaves];
  __shared__ int s_last;

  const int32_t r = static_cast<int32_t>(blockIdx.x) / a.nsplit;
  const int32_t split = static_cast<int32_t>(blockIdx.x) % a.nsplit;
  const int32_t canvas = r / a.canvas_len;
  const int32_t pos = r % a.canvas_len;
  if (a.active != nullptr && a.active[canvas] == 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  // wave index as a scalar, so the batch loop below is uniform control flow
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const float temp = a.temperature[canvas];
  const float c = kLog2e / temp;
  const uint64_t seed = a.seeds[canvas];
  const uint32_t k0 = static_cast<uint32_t>(seed);
  const uint32_t k1 = static_cast<uint32_t>(seed >> 32);
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

  LaneState st;
  // This wave streams supergroups sg_begin + wave, + kWaves, ... in batches of
  // NB stripes. Only the row's last supergroup can be partial, and it is the
  // last one of whichever wave owns it, so the wave's live batches form a
  // flat range [0, n): batch b lies in supergroup sg_of(b) at stripe
  // (b % kBatchesPerSg) * NB, and a block ends after every kBatchesPerSg-th
  // batch and after the last one.
  const int32_t my_sgs = (sg_end - sg_begin - wave + kWaves - 1) / kWaves;
  auto sg_of = [&](int32_t b) { return sg_begin + wave + (b / kBatchesPerSg) * kWaves; };
  auto first_id = [&](int32_t b) {
    return static_cast<int64_t>(sg_of(b)) * kSgIds +
           static_cast<int64_t>(b % kBatchesPerSg) * NB * kStripeIds;
  };
  int32_t n = 0;
  if (my_sgs > 0) {
    const int64_t last_sg_first = static_cast<int64_t>(sg_begin + wave + (my_sgs - 1) * kWaves) * kSgIds;
    const int64_t left = static_cast<int64_t>(vocab) - last_sg_first;  // > 0
    const int64_t live_last = (left + NB * kStripeIds - 1) / (NB * kStripeIds);
    n = (my_sgs - 1) * kBatchesPerSg +
        static_cast<int32_t>(live_last < kBatchesPerSg ? live_last : kBatchesPerSg);
  }
  auto end_of_block = [&](int32_t b) {
    const int32_t j = sg_of(b) * kSlots + lane;
    float score = kNegInf;
    if (st.sb > 0.0) {
      const Words4 rw = philox4x32_10(static_cast<uint32_t>(j), static_cast<uint32_t>(pos),
                                      static_cast<uint32_t>(a.step), kTagBlock, k0, k1);
      score = st.ref + __log2f(static_cast<float>(st.sb)) + kLog2e * gumbel(rw.w[0]);
    }
    if (score > st.best) {  // blocks arrive in increasing j: ties keep the lower
      st.best = score;
      st.bestj = j;
    }
    st.sb = 0.0;
  };
  auto block_ends = [&](int32_t b) { return (b + 1) % kBatchesPerSg == 0 || b + 1 == n; };

  // Byte offset of batch b for this lane; batches past the end point beyond
  // the resource, where buffer loads return zero without touching memory, so
  // every prefetch can be issued unconditionally (a load behind a branch would
  // make the compiler wait for it before reducing the current batch).
  auto byte_of = [&](int32_t b) {
    return b < n ? static_cast<uint32_t>(first_id(b)) * kEB + lane_bytes : kPastEnd;
  };
  uint4 buf0[NB * LPS], buf1[NB * LPS];
  load_batch<kBf16, NB>(buf0, rsrc, byte_of(0));
  for (int32_t b = 0; b < n; b += 2) {
    load_batch<kBf16, NB>(buf1, rsrc, byte_of(b + 1));
    process_batch<kBf16, NB>(buf0, first_id(b) + lane * kSlotIds, first_id(b), vocab, c, st);
    if (block_ends(b)) end_of_block(b);
    load_batch<kBf16, NB>(buf0, rsrc, byte_of(b + 2));
    if (b + 1 < n) {  // a single loop exit keeps the load counters exact
      process_batch<kBf16, NB>(buf1, first_id(b + 1) + lane * kSlotIds, first_id(b + 1), vocab, c, st);
      if (block_ends(b + 1)) end_of_block(b + 1);
    }
  }

  RowPartial wp = wave_partial(st);
  if (lane == 0) s_part[wave] = wp;
  __syncthreads();
  RowPartial p = s_part[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) merge_partial(p, s_part[w]);

  if (a.nsplit > 1) {
    if (tid == 0) {
      a.partials[static_cast<int64_t>(r) * a.nsplit + split] = p;
      __threadfence();
      const uint32_t prev = __hip_atomic_fetch_add(&a.tickets[r], 1u, __ATOMIC_ACQ_REL,
                                                   __HIP_MEMORY_SCOPE_AGENT);
      const int last = (prev == static_cast<uint32_t>(a.nsplit - 1));
      if (last) __hip_atomic_store(&a.tickets[r], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const RowPartial* parts = a.partials + static_cast<int64_t>(r) * a.nsplit;
    p = parts[0];
    for (int sidx = 1; sidx < a.nsplit; ++sidx) merge_partial(p, parts[sidx]);
  }
  finish_row<kBf16>(a, rsrc, r, pos, temp, k0, k1, p);
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
    hipLaunchKernelGGL((canvas_stats_kernel<true, 8>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((canvas_stats_kernel<false, 4>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace dg
