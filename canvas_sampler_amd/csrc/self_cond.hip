// The self-conditioning matmul of the sampling stage: for each row r (a canvas
// position) the expected token embedding under the step's tempered prediction,
//   out[r, n] = sum_v p_r(v) E[v, n],  p_r = softmax(z_r / T),
// in fp32 ("DiffusionGemma: Parallel Denoising From an Autoregressive
// Checkpoint", "Finding": the self-conditioning block feeds the previous
// prediction back; hardware paragraph: the sampling stage runs it with the
// full-vocabulary softmax, in full precision, over the canvas positions).
//
// It is a contraction over the vocabulary (K = V, M = rows, N = d + 1 with the
// normaliser), run on the bf16 matrix cores at fp32 accuracy:
//   - every factor is split exactly into three bf16 parts, x = hi + mid + lo
//     (hi = x with its low 16 bits cleared, mid likewise of x - hi, lo =
//     x - hi - mid, which has at most 8 significant bits), so the product of
//     two factors is the sum of nine exact bf16 x bf16 products; the six whose
//     weight is at least 2^-16 of the leading one are kept (the dropped three
//     are below about 2^-23 of the product, under one fp32 rounding), and
//     v_mfma_f32_32x32x16_bf16 sums them in fp32. Six bf16 products cost
//     less than a third of one fp32 matrix-core product on this chip;
//   - a workgroup owns 256 rows (8 waves x 32) and a slice of the vocabulary;
//   - per 64-id chunk (four 16-id k-steps) the workgroup loads its 256 rows'
//     64 logits with whole 128-byte lines per row and instruction (8 lanes per
//     row), stages them in a padded LDS tile and reads them back in matrix
//     layout: lane l takes row l % 32, ids 16 t + 8 (l / 32) + 0..7 of k-step
//     t, one 16-byte read; it turns them into e = 2^(z c - zmax c),
//     c = log2(e)/T, with zmax the row's largest logit (read at the argmax
//     the statistics pass found), so e <= 1;
//   - the chunk's 64 embedding rows are split and staged once per workgroup
//     in LDS, transposed (column n's 64 values contiguous, three parts), as 32
//     columns: E[v, 0..d-1], a column of ones at d (its sum is the normaliser
//     S = sum_v e_v) and zeros above;
//   - one slice per row tile: the workgroup divides by S and writes out;
//     otherwise it writes its unnormalised partial tile, and a second kernel
//     sums the slices in a fixed order and divides.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace dg {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2eSc = 1.4426950408889634f;
constexpr int kScChunk = 64;
constexpr int kScSteps = kScChunk / 16;     // k-steps of 16 ids per chunk
constexpr int kScBRow = kScChunk + 8;      // bf16 per LDS row (padding spreads the banks)

template <bool kBf16>
__device__ __forceinline__ float logit_at(const void* base, int64_t i) {
  if constexpr (kBf16) {
    const uint16_t b = static_cast<const uint16_t*>(base)[i];
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  } else {
    return static_cast<const float*>(base)[i];
  }
}

// Geometry of the staged logits tile of one chunk: 256 rows of 64 ids, each
// row padded by 16 bytes so that the 16-byte matrix-layout reads of 8
// consecutive rows fall on distinct banks.
template <bool kBf16>
struct ZTile {
  static constexpr int kElem = kBf16 ? 2 : 4;
  static constexpr int kRowBytes = kScChunk * kElem;
  static constexpr int kStride = kRowBytes + 16;
  static constexpr int kPiecesPerRow = kRowBytes / 16;
  static constexpr int kPerPiece = 16 / kElem;
  static constexpr int kPieces = kScRowTile * kPiecesPerRow / kScThreads;  // per thread
  static constexpr int kBytes = kScRowTile * kStride;
};

// f(std::integral_constant<int, i>) for i = 0 .. N-1: the indices are
// constants from the start, so that arrays indexed by them stay in registers
// (a loop unrolled later would leave them in scratch memory).
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// Whether `row` takes part: inside the batch and of an active canvas.
__device__ __forceinline__ bool row_live(const SelfCondArgs& a, int32_t row) {
  return row < a.rows && (a.active == nullptr || a.active[row / a.canvas_len] != 0);
}

// (clang vector type, not HIP's uint4 struct: struct copies between address
// spaces become memory copies that keep the array out of registers)
template <bool kBf16>
struct Raw {
  u32x4_t q[ZTile<kBf16>::kPieces];
};

// This thread's pieces of a chunk, loaded with whole lines per row: piece
// p = tid + kScThreads * i is 16-byte piece p % kPiecesPerRow of tile row
// p / kPiecesPerRow. Every load is unconditional, so that all of them are in
// flight at once: rows past the batch are clamped onto the last row and ids
// past the row's stride onto its last piece. What those clamped pieces hold
// never counts: a row that does not take part has zero probability everywhere
// (see the kernel), and ids at or past the slice end are masked where the
// probabilities are formed.
template <bool kBf16>
__device__ __forceinline__ void load_chunk(const SelfCondArgs& a, int32_t row0, int64_t kc, int tid,
                                           Raw<kBf16>& r) {
  using G = ZTile<kBf16>;
  static_for<G::kPieces>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const int piece = tid + kScThreads * i;
    const int32_t row = min(row0 + piece / G::kPiecesPerRow, a.rows - 1);
    int64_t id = kc + static_cast<int64_t>(piece % G::kPiecesPerRow) * G::kPerPiece;
    id = id < a.row_stride - G::kPerPiece ? id : a.row_stride - G::kPerPiece;
    const int64_t off = static_cast<int64_t>(row) * a.row_stride + id;
    if constexpr (kBf16)
      r.q[i] = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(a.logits) + off);
    else
      r.q[i] = *reinterpret_cast<const u32x4_t*>(static_cast<const float*>(a.logits) + off);
  });
}

template <bool kBf16>
__device__ __forceinline__ void store_chunk(uint8_t* s_z, int tid, const Raw<kBf16>& r) {
  using G = ZTile<kBf16>;
  static_for<G::kPieces>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const int piece = tid + kScThreads * i;
    *reinterpret_cast<u32x4_t*>(s_z + (piece / G::kPiecesPerRow) * G::kStride + (piece % G::kPiecesPerRow) * 16) =
        r.q[i];
  });
}

// The 8 logits of k-step t of tile row `trow` for this half-wave, as fp32.
template <bool kBf16>
__device__ __forceinline__ void read_step(const uint8_t* s_z, int trow, int half, int t, float (&z)[8]) {
  using G = ZTile<kBf16>;
  const uint8_t* base = s_z + trow * G::kStride + (16 * t + 8 * half) * G::kElem;
  if constexpr (kBf16) {
    const uint4 w = *reinterpret_cast<const uint4*>(base);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      z[2 * h] = __uint_as_float(u[h] << 16);
      z[2 * h + 1] = __uint_as_float(u[h] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      const uint4 w = *reinterpret_cast<const uint4*>(base + 16 * g);
      z[4 * g + 0] = __uint_as_float(w.x);
      z[4 * g + 1] = __uint_as_float(w.y);
      z[4 * g + 2] = __uint_as_float(w.z);
      z[4 * g + 3] = __uint_as_float(w.w);
    }
  }
}

// Exact three-part split of an fp32 value x = hi + mid + lo into bf16 values,
// each given as the fp32 pattern whose high 16 bits are that bf16: hi is x
// truncated to its top 16 bits, mid likewise of r1 = x - hi, and lo = r1 - mid
// (at most 8 significant bits, so its low 16 bits are already zero).
struct Split3 {
  uint32_t hi, mid, lo;
};

__device__ __forceinline__ Split3 split3(float x) {
  const uint32_t xb = __float_as_uint(x);
  const float r1 = x - __uint_as_float(xb & 0xFFFF0000u);
  const uint32_t r1b = __float_as_uint(r1);
  const float r2 = r1 - __uint_as_float(r1b & 0xFFFF0000u);
  return Split3{xb, r1b, __float_as_uint(r2)};
}

// The bf16 halves of a and b packed as elements (a, b): one byte permute.
__device__ __forceinline__ uint32_t pack2(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// The chunk's embedding tile as this thread stages it: column n = t % 32,
// ids kc + 4 (t / 32) .. +3 (E[v, n] below d, ones at d, zeros above). The
// loads are unconditional, with ids clamped onto the last embedding row:
// ids at or past the slice end get zero probability.
__device__ __forceinline__ void load_embed(const SelfCondArgs& a, int64_t kc, int tid, float (&ev)[4]) {
  const int n = tid & 31;
  const int nc = n < a.d ? n : a.d - 1;
  static_for<4>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    int64_t v = kc + 4 * (tid >> 5) + i;
    v = v < a.vocab ? v : a.vocab - 1;
    const float e = a.embed[v * a.d + nc];
    ev[i] = n < a.d ? e : (n == a.d ? 1.0f : 0.0f);
  });
}

template <bool kBf16>
__global__ __launch_bounds__(kScThreads) void self_cond_kernel(SelfCondArgs a) {
  static_assert(kScThreads == 32 * (kScChunk / 4), "embedding staging covers the tile once");
  using G = ZTile<kBf16>;
  // LDS slots of the staged tiles: two for bf16 logits; fp32 tiles are twice
  // as large and take one (160 KiB per CU)
  constexpr int kZSlots = kBf16 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) uint8_t s_z[kZSlots][G::kBytes];
  __shared__ __attribute__((aligned(16))) uint16_t s_b[kZSlots][3][32 * kScBRow];
  const int32_t tile = static_cast<int32_t>(blockIdx.x) / a.nslice;
  const int32_t slice = static_cast<int32_t>(blockIdx.x) % a.nslice;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t row0 = tile * kScRowTile;
  const int trow = wave * 32 + (lane & 31);  // this lane's row in the tile
  const int32_t row = row0 + trow;

  // rows past the batch or of inactive canvases get zmax*c = +inf, so that
  // every probability of theirs is exactly 0 whatever their tile holds
  float c = 1.0f, mc = __builtin_inff();
  if (row_live(a, row)) {
    const int64_t off = static_cast<int64_t>(row) * a.row_stride;
    int32_t am = a.argmax[row];
    am = am < 0 ? 0 : (am >= a.vocab ? a.vocab - 1 : am);
    c = kLog2eSc / a.temperature[row / a.canvas_len];
    mc = logit_at<kBf16>(a.logits, off + am) * c;
  }
  const int64_t k_begin = static_cast<int64_t>(slice) * a.kslice;
  const int64_t k_end = k_begin + a.kslice < a.vocab ? k_begin + a.kslice : a.vocab;

  // software pipeline: chunk i + 2 is loaded into registers while chunk i is
  // multiplied out of LDS. With two LDS slots one barrier per chunk both
  // publishes chunk i and retires the reads of chunk i - 1 (whose slot chunk
  // i + 1 takes next); with one slot a second barrier guards the slot.
  Raw<kBf16> raw0, raw1;
  float ev0[4], ev1[4];
  load_chunk<kBf16>(a, row0, k_begin, tid, raw0);
  load_embed(a, k_begin, tid, ev0);
  if (k_begin + kScChunk < k_end) {
    load_chunk<kBf16>(a, row0, k_begin + kScChunk, tid, raw1);
    load_embed(a, k_begin + kScChunk, tid, ev1);
  }
  f32x16_t acc0 = {}, acc1 = {};
  const int sn = tid & 31, sk = 4 * (tid >> 5);
  const int bo = (lane & 31) * kScBRow + 8 * half;
  // kTail: the slice's last chunk reaches past its end; ids there get zero
  // probability
  auto run_chunk = [&](auto slot, auto tail, int64_t kc, Raw<kBf16>& raw, float(&ev)[4])
                       __attribute__((always_inline)) {
    constexpr int S = decltype(slot)::value;
    constexpr bool kTail = decltype(tail)::value;
    constexpr int Z = kZSlots == 2 ? S : 0;
    uint8_t* zb = s_z[Z];
    uint16_t(*bb)[32 * kScBRow] = s_b[Z];
    if constexpr (kZSlots == 1) __syncthreads();  // the previous chunk's LDS reads are done
    store_chunk<kBf16>(zb, tid, raw);
    {  // this chunk's embedding parts: 4 consecutive ids of one column
      const Split3 e0 = split3(ev[0]), e1 = split3(ev[1]), e2 = split3(ev[2]), e3 = split3(ev[3]);
      const int o = sn * kScBRow + sk;
      *reinterpret_cast<uint2*>(&bb[0][o]) = make_uint2(pack2(e0.hi, e1.hi), pack2(e2.hi, e3.hi));
      *reinterpret_cast<uint2*>(&bb[1][o]) = make_uint2(pack2(e0.mid, e1.mid), pack2(e2.mid, e3.mid));
      *reinterpret_cast<uint2*>(&bb[2][o]) = make_uint2(pack2(e0.lo, e1.lo), pack2(e2.lo, e3.lo));
    }
    const int64_t kn = kc + 2 * kScChunk;
    if (kn < k_end) {
      load_chunk<kBf16>(a, row0, kn, tid, raw);
      load_embed(a, kn, tid, ev);
    }
    __syncthreads();  // chunk kc is in LDS (and, with two slots, every wave is done with the chunk before it)
    // this lane's 8 factors of k-step t, split into three parts
    auto factors = [&](int t, bf16x8_t& xh, bf16x8_t& xm, bf16x8_t& xl) __attribute__((always_inline)) {
      float z[8];
      read_step<kBf16>(zb, trow, half, t, z);
      uint32_t h[8], m[8], l[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf(z[j], c, -mc));
        if constexpr (kTail) e = kc + 16 * t + 8 * half + j < k_end ? e : 0.0f;
        const Split3 sp = split3(e);
        h[j] = sp.hi;
        m[j] = sp.mid;
        l[j] = sp.lo;
      }
      xh = as_bf16x8(u32x4_t{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])});
      xm = as_bf16x8(u32x4_t{pack2(m[0], m[1]), pack2(m[2], m[3]), pack2(m[4], m[5]), pack2(m[6], m[7])});
      xl = as_bf16x8(u32x4_t{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])});
    };
    // the factors of k-step t + 1 are formed while the matrix cores take the
    // products of step t: the six products are spread through that VALU work
    bf16x8_t xh, xm, xl;
    factors(0, xh, xm, xl);
#pragma unroll
    for (int t = 0; t < kScSteps; ++t) {
      const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(&bb[0][bo + 16 * t]);
      const bf16x8_t bm = *reinterpret_cast<const bf16x8_t*>(&bb[1][bo + 16 * t]);
      const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(&bb[2][bo + 16 * t]);
      bf16x8_t nh = xh, nm = xm, nl = xl;
      if (t + 1 < kScSteps) factors(t + 1, nh, nm, nl);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl, bh, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xm, bm, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, bl, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xm, bh, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, bm, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, bh, acc1, 0, 0, 0);
      if (t + 1 < kScSteps) {
#pragma unroll
        for (int k = 0; k < 6; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one matrix-core product
          __builtin_amdgcn_sched_group_barrier(0x002, 12, 0);  // then VALU work of the next step
        }
      }
      xh = nh;
      xm = nm;
      xl = nl;
    }
  };
  // chunk i of the slice takes register slot i % 2: a loop over pairs of
  // whole chunks keeps every slot index a constant; then at most one whole
  // chunk and the partial one
  using Slot0 = std::integral_constant<int, 0>;
  using Slot1 = std::integral_constant<int, 1>;
  using Full = std::integral_constant<bool, false>;
  using Tail = std::integral_constant<bool, true>;
  const int64_t full_end = k_begin + (k_end - k_begin) / kScChunk * kScChunk;
  int64_t kc = k_begin;
  for (; kc + kScChunk < full_end; kc += 2 * kScChunk) {
    run_chunk(Slot0{}, Full{}, kc, raw0, ev0);
    run_chunk(Slot1{}, Full{}, kc + kScChunk, raw1, ev1);
  }
  if (kc < full_end) {
    run_chunk(Slot0{}, Full{}, kc, raw0, ev0);
    if (kc + kScChunk < k_end) run_chunk(Slot1{}, Tail{}, kc + kScChunk, raw1, ev1);
  } else if (kc < k_end) {
    run_chunk(Slot0{}, Tail{}, kc, raw0, ev0);
  }
  const f32x16_t acc = acc0 + acc1;
  // lane l, register r holds D[i][n] with n = l % 32 and
  // i = 8 (r / 4) + 4 (l / 32) + r % 4 (the 32x32 fp32 accumulator layout)
  const int n = lane & 31;
  const int32_t wrow0 = row0 + wave * 32;
  if (a.nslice == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float s = __shfl(acc[r], (lane & 32) | a.d);  // the normaliser of this row
      const int32_t gr = wrow0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (n < a.d && row_live(a, gr)) a.out[static_cast<int64_t>(gr) * a.d + n] = acc[r] / s;
    }
  } else {
    float* part = a.partials + static_cast<int64_t>(slice) * a.rows_pad * 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int32_t gr = wrow0 + 8 * (r >> 2) + 4 * half + (r & 3);
      part[static_cast<int64_t>(gr) * 32 + n] = acc[r];
    }
  }
}

// out[r, n] = (sum over slices of partial[s][r][n]) / (same for column d).
// One workgroup per row: thread t takes columns 4 (t % 8) .. +3 of the slices
// s = 16 g .. 16 g + 15 of group g = t / 8 (32 groups of 16 slices at a
// time, more rounds when there are more slices), then the groups' sums are
// combined in LDS in group order, so the result does not depend on timing.
__global__ __launch_bounds__(256) void self_cond_reduce_kernel(SelfCondArgs a) {
  __shared__ float4 s_part[32][8];
  const int32_t r = static_cast<int32_t>(blockIdx.x);
  if (a.active != nullptr && a.active[r / a.canvas_len] == 0) return;  // uniform over the workgroup
  const int t = threadIdx.x, quad = t & 7, group = t >> 3;
  const int64_t stride = static_cast<int64_t>(a.rows_pad) * 32;
  const float* base = a.partials + static_cast<int64_t>(r) * 32 + 4 * quad;
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int32_t s0 = 16 * group; s0 < a.nslice; s0 += 16 * 32) {
    float4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
      v[i] = s0 + i < a.nslice ? *reinterpret_cast<const float4*>(base + (s0 + i) * stride)
                               : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      sum.x += v[i].x;
      sum.y += v[i].y;
      sum.z += v[i].z;
      sum.w += v[i].w;
    }
  }
  s_part[group][quad] = sum;
  __syncthreads();
  if (t < 32) {
    float tot = 0.0f, den = 0.0f;
    for (int g = 0; g < 32; ++g) {
      const float4 q = s_part[g][t >> 2];
      const float4 qd = s_part[g][a.d >> 2];
      const int k = t & 3, kd = a.d & 3;
      tot += k == 0 ? q.x : k == 1 ? q.y : k == 2 ? q.z : q.w;
      den += kd == 0 ? qd.x : kd == 1 ? qd.y : kd == 2 ? qd.z : qd.w;
    }
    if (t < a.d) a.out[static_cast<int64_t>(r) * a.d + t] = tot / den;
  }
}

}  // namespace

void choose_self_cond_slices(int32_t rows, int32_t vocab, int32_t* nslice, int32_t* kslice) {
  const int32_t tiles = (rows + kScRowTile - 1) / kScRowTile;
  const int32_t target = kScTargetWorkgroups / tiles;
  if (target <= 1) {
    *nslice = 1;
    *kslice = vocab;
    return;
  }
  int64_t ks = (static_cast<int64_t>(vocab) + target - 1) / target;
  ks = (ks + kScChunk - 1) / kScChunk * kScChunk;
  *kslice = static_cast<int32_t>(ks);
  *nslice = static_cast<int32_t>((vocab + ks - 1) / ks);
}

hipError_t launch_self_cond(const SelfCondArgs& a, bool bf16, hipStream_t stream) {
  const int32_t tiles = (a.rows + kScRowTile - 1) / kScRowTile;
  const dim3 grid(static_cast<unsigned>(tiles) * static_cast<unsigned>(a.nslice));
  if (bf16)
    hipLaunchKernelGGL(self_cond_kernel<true>, grid, dim3(kScThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(self_cond_kernel<false>, grid, dim3(kScThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nslice == 1) return e;
  hipLaunchKernelGGL(self_cond_reduce_kernel, dim3(static_cast<unsigned>(a.rows)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace dg
