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

// This thread's pieces of a chunk, loaded with whole lines per row: piece
// p = tid + kScThreads * i is 16-byte piece p % kPiecesPerRow of tile row
// p / kPiecesPerRow. Rows past the batch or of inactive canvases, and ids at or past `end`, read as
// -inf, so their probability is exactly 0 and no later step needs a bound
// check; only a piece that straddles `end` (V not a multiple of the piece) is
// masked element by element. Pieces never cross the row's padded end: the row
// stride is a multiple of 16 bytes and every piece that is read starts below
// `end` <= V.
// Whether `row` takes part: inside the batch and of an active canvas.
__device__ __forceinline__ bool row_live(const SelfCondArgs& a, int32_t row) {
  return row < a.rows && (a.active == nullptr || a.active[row / a.canvas_len] != 0);
}

template <bool kBf16>
struct Raw {
  uint4 q[ZTile<kBf16>::kPieces];
};

template <bool kBf16>
__device__ __forceinline__ void load_chunk(const SelfCondArgs& a, int32_t row0, int64_t kc, int64_t end,
                                           int tid, Raw<kBf16>& r) {
  using G = ZTile<kBf16>;
  constexpr uint32_t kNegInf2 = kBf16 ? 0xFF80FF80u : 0xFF800000u;  // one 32-bit word of -inf
#pragma unroll
  for (int i = 0; i < G::kPieces; ++i) {
    const int piece = tid + kScThreads * i;
    const int32_t row = row0 + piece / G::kPiecesPerRow;
    const int64_t id = kc + static_cast<int64_t>(piece % G::kPiecesPerRow) * G::kPerPiece;
    uint4 w = make_uint4(kNegInf2, kNegInf2, kNegInf2, kNegInf2);
    if (row_live(a, row) && id < end) {
      const int64_t off = static_cast<int64_t>(row) * a.row_stride + id;
      if constexpr (kBf16)
        w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.logits) + off);
      else
        w = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.logits) + off);
      if (id + G::kPerPiece > end) {  // the piece that straddles the end of the row
        uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < G::kPerPiece; ++e) {
          if (id + e < end) continue;
          if constexpr (kBf16)
            u[e >> 1] = (e & 1) ? (u[e >> 1] & 0x0000FFFFu) | 0xFF800000u : (u[e >> 1] & 0xFFFF0000u) | 0xFF80u;
          else
            u[e] = 0xFF800000u;
        }
        w = make_uint4(u[0], u[1], u[2], u[3]);
      }
    }
    r.q[i] = w;
  }
}

template <bool kBf16>
__device__ __forceinline__ void store_chunk(uint8_t* s_z, int tid, const Raw<kBf16>& r) {
  using G = ZTile<kBf16>;
#pragma unroll
  for (int i = 0; i < G::kPieces; ++i) {
    const int piece = tid + kScThreads * i;
    *reinterpret_cast<uint4*>(s_z + (piece / G::kPiecesPerRow) * G::kStride + (piece % G::kPiecesPerRow) * 16) =
        r.q[i];
  }
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
// ids kc + 4 (t / 32) .. +3, each split into its three parts.
__device__ __forceinline__ void load_embed(const SelfCondArgs& a, int64_t kc, int64_t k_end, int tid,
                                           float (&ev)[4]) {
  const int n = tid & 31;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t v = kc + 4 * (tid >> 5) + i;
    float e = 0.0f;
    if (v < k_end) e = n < a.d ? a.embed[v * a.d + n] : (n == a.d ? 1.0f : 0.0f);
    ev[i] = e;
  }
}

template <bool kBf16>
__global__ __launch_bounds__(kScThreads) void self_cond_kernel(SelfCondArgs a) {
  static_assert(kScThreads == 32 * (kScChunk / 4), "embedding staging covers the tile once");
  using G = ZTile<kBf16>;
  __shared__ __attribute__((aligned(16))) uint8_t s_z[G::kBytes];
  __shared__ __attribute__((aligned(16))) uint16_t s_b[3][32 * kScBRow];
  const int32_t tile = static_cast<int32_t>(blockIdx.x) / a.nslice;
  const int32_t slice = static_cast<int32_t>(blockIdx.x) % a.nslice;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t row0 = tile * kScRowTile;
  const int trow = wave * 32 + (lane & 31);  // this lane's row in the tile
  const int32_t row = row0 + trow;

  // rows past the batch or of inactive canvases are all -inf in the tile:
  // with c = 1 and zmax*c = 0 their probabilities are exactly 0
  float c = 1.0f, mc = 0.0f;
  if (row_live(a, row)) {
    const int64_t off = static_cast<int64_t>(row) * a.row_stride;
    int32_t am = a.argmax[row];
    am = am < 0 ? 0 : (am >= a.vocab ? a.vocab - 1 : am);
    c = kLog2eSc / a.temperature[row / a.canvas_len];
    mc = logit_at<kBf16>(a.logits, off + am) * c;
  }
  const int64_t k_begin = static_cast<int64_t>(slice) * a.kslice;
  const int64_t k_end = k_begin + a.kslice < a.vocab ? k_begin + a.kslice : a.vocab;

  // software pipeline: chunk i + 1 is loaded into registers while chunk i is
  // multiplied out of LDS; two barriers per chunk guard the single LDS tiles
  Raw<kBf16> raw;
  float ev[4];
  load_chunk<kBf16>(a, row0, k_begin, k_end, tid, raw);
  load_embed(a, k_begin, k_end, tid, ev);
  f32x16_t acc0 = {}, acc1 = {};
  const int sn = tid & 31, sk = 4 * (tid >> 5);
  const int bo = (lane & 31) * kScBRow + 8 * half;
  for (int64_t kc = k_begin; kc < k_end; kc += kScChunk) {
    __syncthreads();  // the previous chunk's LDS reads are done
    store_chunk<kBf16>(s_z, tid, raw);
    {  // this chunk's embedding parts: 4 consecutive ids of one column
      const Split3 e0 = split3(ev[0]), e1 = split3(ev[1]), e2 = split3(ev[2]), e3 = split3(ev[3]);
      const int o = sn * kScBRow + sk;
      *reinterpret_cast<uint2*>(&s_b[0][o]) = make_uint2(pack2(e0.hi, e1.hi), pack2(e2.hi, e3.hi));
      *reinterpret_cast<uint2*>(&s_b[1][o]) = make_uint2(pack2(e0.mid, e1.mid), pack2(e2.mid, e3.mid));
      *reinterpret_cast<uint2*>(&s_b[2][o]) = make_uint2(pack2(e0.lo, e1.lo), pack2(e2.lo, e3.lo));
    }
    const int64_t kn = kc + kScChunk;
    if (kn < k_end) {
      load_chunk<kBf16>(a, row0, kn, k_end, tid, raw);
      load_embed(a, kn, k_end, tid, ev);
    }
    __syncthreads();  // this chunk's tiles are in LDS
#pragma unroll
    for (int t = 0; t < kScSteps; ++t) {
      // this lane's 8 factors of k-step t, split into three parts
      float z[8];
      read_step<kBf16>(s_z, trow, half, t, z);
      uint32_t h[8], m[8], l[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const Split3 sp = split3(__builtin_amdgcn_exp2f(__builtin_fmaf(z[j], c, -mc)));
        h[j] = sp.hi;
        m[j] = sp.mid;
        l[j] = sp.lo;
      }
      const bf16x8_t xh = as_bf16x8(u32x4_t{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]),
                                            pack2(h[6], h[7])});
      const bf16x8_t xm = as_bf16x8(u32x4_t{pack2(m[0], m[1]), pack2(m[2], m[3]), pack2(m[4], m[5]),
                                            pack2(m[6], m[7])});
      const bf16x8_t xl = as_bf16x8(u32x4_t{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]),
                                            pack2(l[6], l[7])});
      const bf16x8_t bh = *reinterpret_cast<const bf16x8_t*>(&s_b[0][bo + 16 * t]);
      const bf16x8_t bm = *reinterpret_cast<const bf16x8_t*>(&s_b[1][bo + 16 * t]);
      const bf16x8_t bl = *reinterpret_cast<const bf16x8_t*>(&s_b[2][bo + 16 * t]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xl, bh, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xm, bm, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, bl, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xm, bh, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, bm, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xh, bh, acc1, 0, 0, 0);
    }
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
