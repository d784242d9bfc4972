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
//   - per 64-id chunk (four 16-id k-steps) each wave loads its own 32 rows'
//     64 logits with whole 128-byte lines per row and instruction (8 lanes per
//     row), stages them in its own padded LDS tile and reads them back in
//     matrix layout: lane l takes row l % 32, ids 16 t + 8 (l / 32) + 0..7 of
//     k-step t, one 16-byte read; it turns them into e = 2^(z c - zmax c),
//     c = log2(e)/T, with zmax the row's largest logit (read at the argmax
//     the statistics pass found), so e <= 1. No wave waits for another's
//     tile;
//   - the embedding rows of four chunks (two for fp32 logits) are split and
//     staged together in LDS, transposed (column n's 64 values of a chunk
//     contiguous, three parts), as 32 columns: E[v, 0..d-1], a column of ones
//     at d (its sum is the normaliser S = sum_v e_v) and zeros above, and
//     zeros for ids past the slice; the workgroup meets at one barrier per
//     such group;
//   - every load is a buffer load issued on every path, its resource ending
//     where the data ends (rows past the batch and ids past the slice read
//     zeros), so each wait is for exactly the data it needs: the next
//     group's embedding and the chunks two and three ahead stay in flight
//     while a chunk is multiplied; ids past the vocabulary (the row's
//     padding) are set to -inf in the one chunk that holds any;
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

// Geometry of one wave's staged logits tile of a chunk: the wave's 32 rows of
// 64 ids, each row padded by 16 bytes so that the 16-byte matrix-layout reads
// of 8 consecutive rows fall on distinct banks. The wave loads, stores and
// reads its own tile, so no other wave waits for it.
template <bool kBf16>
struct ZTile {
  static constexpr int kElem = kBf16 ? 2 : 4;
  static constexpr int kRowBytes = kScChunk * kElem;
  static constexpr int kStride = kRowBytes + 16;
  static constexpr int kPiecesPerRow = kRowBytes / 16;
  static constexpr int kPerPiece = 16 / kElem;
  static constexpr int kPieces = 32 * kPiecesPerRow / 64;  // 16-byte pieces per lane
  static constexpr int kBytes = 32 * kStride;
  // chunks per staged embedding group: the workgroup meets at one barrier per
  // group (two LDS slots of kGroup chunks; fp32 tiles leave room for two)
  static constexpr int kGroup = kBf16 ? 4 : 2;
};

// One chunk's embedding tile in LDS: three bf16 parts of 32 columns, each
// column's 64 values contiguous (padded to kScBRow).
constexpr int kEChunk = 3 * 32 * kScBRow;

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

// The wave's 32 logits rows through one buffer resource based at its first
// row; its records end with the batch's last row, so rows past the batch
// read zeros (they never count: see the kernel). The 32 rows' bytes stay
// below 4 GiB (the entry points check the row stride).
template <bool kBf16>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const SelfCondArgs& a, int32_t wrow0) {
  constexpr int64_t kElem = ZTile<kBf16>::kElem;
  const int32_t left = a.rows - wrow0;
  const int64_t nrows = left <= 0 ? 0 : (left >= 32 ? 32 : left);
  const uintptr_t base =
      reinterpret_cast<uintptr_t>(a.logits) + static_cast<uint64_t>(static_cast<int64_t>(wrow0) * a.row_stride * kElem);
  // (the wave's values, kept scalar: the compiler cannot see that every lane
  // holds the same)
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(base));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(base >> 32));
  const uint32_t num = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(nrows * a.row_stride * kElem));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo), 0,
                                           static_cast<int>(num), 0x00020000);
}

// This lane's pieces of a chunk of the wave's rows, loaded with whole lines
// per row and instruction: piece p = lane + 64 i is 16-byte piece
// p % kPiecesPerRow of wave row p / kPiecesPerRow, at byte offset
// loff + i * step + kc * size (loff = the lane's offset of piece `lane` at id
// 0, step = the bytes of the rows that 64 pieces span). Every load is issued
// on every path, so each wait is for exactly the chunk it needs. Ids past
// the row's end read the next row's values or zeros; they are past the
// vocabulary, and the chunk that holds them is masked before it is staged.
template <bool kBf16>
__device__ __forceinline__ void load_chunk(__amdgpu_buffer_rsrc_t rows, uint32_t loff, uint32_t step, int64_t kc,
                                           Raw<kBf16>& r) {
  using G = ZTile<kBf16>;
  const uint32_t kb = static_cast<uint32_t>(kc) * G::kElem;
  static_for<G::kPieces>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    r.q[i] = __builtin_amdgcn_raw_buffer_load_b128(rows, loff + (i * step + kb), 0, 0);
  });
}

template <bool kBf16>
__device__ __forceinline__ void store_chunk(uint8_t* s_z, int lane, const Raw<kBf16>& r) {
  using G = ZTile<kBf16>;
  static_for<G::kPieces>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const int piece = lane + 64 * i;
    *reinterpret_cast<u32x4_t*>(s_z + (piece / G::kPiecesPerRow) * G::kStride + (piece % G::kPiecesPerRow) * 16) =
        r.q[i];
  });
}

// In the wave's staged tile of the chunk from id kc, ids at or past the
// vocabulary (only the last chunk of a row holds any) become -inf, so that
// whatever the rows' padding holds, their probabilities are exactly 0. Lane
// l rewrites row l % 32, every other id from the first past the vocabulary.
// (A loop of LDS writes in its own branch: the compiler does not fold it into
// the common path.)
template <bool kBf16>
__device__ __forceinline__ void mask_past_vocab(uint8_t* zw, int64_t kc, int32_t vocab, int lane) {
  using G = ZTile<kBf16>;
  if (kc + kScChunk <= vocab) return;
  const int first = static_cast<int>(vocab - kc);  // a chunk starts inside the vocabulary
  uint8_t* rowp = zw + (lane & 31) * G::kStride;
  for (int id = first + (lane >> 5); id < kScChunk; id += 2) {
    if constexpr (kBf16)
      *reinterpret_cast<uint16_t*>(rowp + 2 * id) = 0xFF80u;
    else
      *reinterpret_cast<uint32_t*>(rowp + 4 * id) = 0xFF800000u;
  }
}

// Exact three-part split of an fp32 value x = hi + mid + lo into bf16 values,
// each given as the fp32 pattern whose high 16 bits are that bf16: hi is x
// truncated to its top 16 bits, mid likewise of r1 = x - hi, and lo = r1 - mid
// (at most 8 significant bits, so its low 16 bits are already zero).
// (A split by the packed bf16 conversion, with the residuals as bf16 dot
// products, takes fewer instructions but runs slower beside the matrix-core
// products: those dot products compete with them.)
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

// The embedding values this thread stages for a group of kGroup chunks from
// id kg: column n = tid % 32 (clamped onto column d - 1; the staging puts the
// ones and zeros above d), ids kg + 64 c + 4 (tid / 32) .. +3 of chunk c.
// Chunk c is read through a buffer resource of its own, based at its first
// row and holding its rows before the slice end (none for a chunk past it),
// so ids at or past the slice end read zeros, at the thread's fixed offsets
// voff[i] = ((4 (tid / 32) + i) d + n) * 4 bytes: no per-load address
// arithmetic, and every load is issued on every path.
template <int kG>
__device__ __forceinline__ void load_embed(const SelfCondArgs& a, int64_t kg, int64_t k_end, const uint32_t (&voff)[4],
                                           float (&ev)[kG][4]) {
  static_for<kG>([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    const int64_t k0 = kg + 64 * c;
    const int64_t left = k_end - k0;
    const int32_t nrows = left <= 0 ? 0 : (left >= 64 ? 64 : static_cast<int32_t>(left));
    const __amdgpu_buffer_rsrc_t rsrc =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.embed) + k0 * a.d, 0, nrows * a.d * 4, 0x00020000);
    static_for<4>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      ev[c][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc, voff[i], 0, 0));
    });
  });
}

// Stages a group's embedding tiles: E[v, n] below d, ones at d, zeros above,
// and zeros for ids at or past the slice end (so that the probabilities
// formed there, from clamped or neighbouring logits, never count), split into
// three parts, column n's 4 ids as one 8-byte write per part. The loads read
// zeros past the slice end; only the ones column tests the ids there, and
// only in the group that reaches past it.
template <int kG, typename X>
__device__ __forceinline__ void stage_parts(uint16_t* eb, int tid, X&& value) {
  const int n = tid & 31, sk = 4 * (tid >> 5);
  static_for<kG>([&](auto cc) {
    constexpr int c = decltype(cc)::value;
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = value(c, i);
    const Split3 e0 = split3(x[0]), e1 = split3(x[1]), e2 = split3(x[2]), e3 = split3(x[3]);
    uint16_t* b = eb + c * kEChunk + n * kScBRow + sk;
    *reinterpret_cast<uint2*>(b) = make_uint2(pack2(e0.hi, e1.hi), pack2(e2.hi, e3.hi));
    *reinterpret_cast<uint2*>(b + 32 * kScBRow) = make_uint2(pack2(e0.mid, e1.mid), pack2(e2.mid, e3.mid));
    *reinterpret_cast<uint2*>(b + 64 * kScBRow) = make_uint2(pack2(e0.lo, e1.lo), pack2(e2.lo, e3.lo));
  });
}

template <int kG>
__device__ __forceinline__ void stage_embed(uint16_t* eb, const SelfCondArgs& a, int64_t kg, int64_t k_end, int tid,
                                            const float (&ev)[kG][4]) {
  const int n = tid & 31, sk = 4 * (tid >> 5);
  const bool data = n < a.d;
  const float one = n == a.d ? 1.0f : 0.0f;
  if (kg + 64 * kG <= k_end) {
    stage_parts<kG>(eb, tid, [&](int c, int i) { return data ? ev[c][i] : one; });
  } else {
    const int32_t lim = static_cast<int32_t>(k_end - kg) - sk;  // ids 64 c + i below lim count
    stage_parts<kG>(eb, tid, [&](int c, int i) { return data ? ev[c][i] : (64 * c + i < lim ? one : 0.0f); });
  }
}

template <bool kBf16>
__global__ __launch_bounds__(kScThreads) void self_cond_kernel(SelfCondArgs a) {
  static_assert(kScThreads == 32 * (kScChunk / 4), "embedding staging covers a chunk's tile once");
  using G = ZTile<kBf16>;
  constexpr int kG = G::kGroup;
  static_assert(kG % 2 == 0, "a group holds whole pairs of chunks (two register slots)");
  __shared__ __attribute__((aligned(16))) uint8_t s_z[kScThreads / 64][G::kBytes];
  __shared__ __attribute__((aligned(16))) uint16_t s_b[2][kG * kEChunk];
  const int32_t tile = static_cast<int32_t>(blockIdx.x) / a.nslice;
  const int32_t slice = static_cast<int32_t>(blockIdx.x) % a.nslice;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t row0 = tile * kScRowTile;
  const int32_t wrow0 = row0 + wave * 32;
  const int wr = lane & 31;  // this lane's row among the wave's 32
  const int32_t row = wrow0 + wr;
  uint8_t* zw = s_z[wave];

  const int64_t k_begin = static_cast<int64_t>(slice) * a.kslice;
  const int64_t k_end = k_begin + a.kslice < a.vocab ? k_begin + a.kslice : a.vocab;
  const int32_t nch = static_cast<int32_t>((k_end - k_begin + kScChunk - 1) / kScChunk);
  const int32_t ngroups = (nch + kG - 1) / kG;
  // chunk and group starts; past the slice they repeat the last one (loads
  // that hit the cache and are never used), so every load is issued
  auto kc_of = [&](int32_t j) { return k_begin + static_cast<int64_t>(j < nch ? j : nch - 1) * kScChunk; };
  auto kg_of = [&](int32_t g) {
    return k_begin + static_cast<int64_t>(g < ngroups ? g : ngroups - 1) * kG * kScChunk;
  };

  // the row's constants, through buffer resources like every other load
  // (a row past the batch reads zeros, and so does the flag without a flag
  // array): its argmax, temperature and canvas flag first, the logit at the
  // argmax once the argmax is in, behind the pipeline's first loads. The flag
  // is read through the aligned 32-bit word that holds it.
  const int32_t ncanvas = (a.rows + a.canvas_len - 1) / a.canvas_len;
  const int32_t canvas = row / a.canvas_len;
  const uint32_t fmis = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(a.active) & 3u);
  const __amdgpu_buffer_rsrc_t r_flag = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a.active) - fmis, 0, a.active != nullptr ? static_cast<int>((fmis + ncanvas + 3) & ~3u) : 0,
      0x00020000);
  const __amdgpu_buffer_rsrc_t r_am =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<int32_t*>(a.argmax), 0, a.rows * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t r_temp =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(a.temperature), 0, ncanvas * 4, 0x00020000);
  const uint32_t fbyte = fmis + static_cast<uint32_t>(canvas);
  const uint32_t fword = __builtin_amdgcn_raw_buffer_load_b32(r_flag, fbyte & ~3u, 0, 0);
  int32_t am = static_cast<int32_t>(__builtin_amdgcn_raw_buffer_load_b32(r_am, static_cast<uint32_t>(row) * 4, 0, 0));
  const float temp = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r_temp, static_cast<uint32_t>(canvas) * 4, 0, 0));

  // software pipeline: the embedding of group g + 1 and chunk j + 2 are in
  // flight in registers while chunk j is multiplied
  // (in this order: the scheduler barriers keep each wait exact)
  const __amdgpu_buffer_rsrc_t rows = rows_rsrc<kBf16>(a, wrow0);
  const uint32_t loff = static_cast<uint32_t>(
      ((lane / G::kPiecesPerRow) * a.row_stride + (lane % G::kPiecesPerRow) * G::kPerPiece) * G::kElem);
  const uint32_t lstep = static_cast<uint32_t>((64 / G::kPiecesPerRow) * a.row_stride * G::kElem);
  Raw<kBf16> raw0, raw1;
  float ev[kG][4];
  uint32_t voff[4];
  {
    const int en = tid & 31;
    const int nc = en < a.d ? en : a.d - 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) voff[i] = static_cast<uint32_t>(((4 * (tid >> 5) + i) * a.d + nc) * 4);
  }
  __builtin_amdgcn_sched_barrier(0);
  load_embed<kG>(a, kg_of(0), k_end, voff, ev);
  __builtin_amdgcn_sched_barrier(0);
  load_chunk<kBf16>(rows, loff, lstep, kc_of(0), raw0);
  load_chunk<kBf16>(rows, loff, lstep, kc_of(1), raw1);
  __builtin_amdgcn_sched_barrier(0);

  am = am < 0 ? 0 : (am >= a.vocab ? a.vocab - 1 : am);
  const uint32_t zoff = static_cast<uint32_t>((wr * a.row_stride + am) * G::kElem);
  float zmax;
  if constexpr (kBf16)
    zmax = __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(rows, zoff, 0, 0)) << 16);
  else
    zmax = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rows, zoff, 0, 0));
  const uint32_t act = (fword >> (8 * (fbyte & 3u))) & 0xFFu;
  // rows past the batch or of inactive canvases get zmax*c = +inf, so that
  // every probability of theirs is exactly 0 whatever their tile holds
  const bool live = row < a.rows && (a.active == nullptr || act != 0);
  const float c = live ? kLog2eSc / temp : 1.0f;
  const float mc = live ? zmax * c : __builtin_inff();

  f32x16_t acc0 = {}, acc1 = {};
  const int bo = wr * kScBRow + 8 * half;
  // a chunk's operands as this lane reads them from LDS, all at the chunk's
  // start: its row's logits of the four k-steps and the embedding parts of
  // its column, in k-step order (LDS answers a wave in order, so each k-step
  // waits for its own reads only)
  constexpr int kZq = kBf16 ? 1 : 2;  // 16-byte reads of a k-step's 8 logits
  struct Operands {
    u32x4_t z[kScSteps][kZq];
    bf16x8_t b[kScSteps][3];
  };
  auto read_operands = [&](const uint16_t* ec, Operands& o) __attribute__((always_inline)) {
    static_for<kScSteps>([&](auto tc) {
      constexpr int t = decltype(tc)::value;
      const uint8_t* zb = zw + wr * G::kStride + (16 * t + 8 * half) * G::kElem;
#pragma unroll
      for (int q = 0; q < kZq; ++q) o.z[t][q] = *reinterpret_cast<const u32x4_t*>(zb + 16 * q);
#pragma unroll
      for (int p = 0; p < 3; ++p) o.b[t][p] = *reinterpret_cast<const bf16x8_t*>(ec + 32 * kScBRow * p + bo + 16 * t);
    });
  };
  // this lane's 8 factors of k-step t, split into three parts
  auto factors = [&](const Operands& o, int t, bf16x8_t& xh, bf16x8_t& xm, bf16x8_t& xl)
                     __attribute__((always_inline)) {
    float z[8];
    if constexpr (kBf16) {
      const u32x4_t w = o.z[t][0];
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        z[2 * h] = __uint_as_float(w[h] << 16);
        z[2 * h + 1] = __uint_as_float(w[h] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int h = 0; h < 4; ++h) z[4 * q + h] = __uint_as_float(o.z[t][q][h]);
    }
    uint32_t h[8], m[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const Split3 sp = split3(__builtin_amdgcn_exp2f(__builtin_fmaf(z[j], c, -mc)));
      h[j] = sp.hi;
      m[j] = sp.mid;
      l[j] = sp.lo;
    }
    xh = as_bf16x8(u32x4_t{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])});
    xm = as_bf16x8(u32x4_t{pack2(m[0], m[1]), pack2(m[2], m[3]), pack2(m[4], m[5]), pack2(m[6], m[7])});
    xl = as_bf16x8(u32x4_t{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])});
  };
  // the products of one chunk; the factors of k-step t + 1 are formed while
  // the matrix cores take the six products of step t, spread through that
  // VALU work
  auto multiply = [&](const Operands& o) __attribute__((always_inline)) {
    // every LDS read of the chunk first, so that each k-step waits for its own
    __builtin_amdgcn_sched_group_barrier(0x100, kScSteps * (kZq + 3), 0);
    bf16x8_t xh, xm, xl;
    factors(o, 0, xh, xm, xl);
#pragma unroll
    for (int t = 0; t < kScSteps; ++t) {
      bf16x8_t nh = xh, nm = xm, nl = xl;
      if (t + 1 < kScSteps) factors(o, t + 1, nh, nm, nl);
      const bf16x8_t bh = o.b[t][0], bm = o.b[t][1], bl = o.b[t][2];
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

  // The wave's tile holds chunk 0 before the first group; chunk 2 goes into
  // its register slot.
  store_chunk<kBf16>(zw, lane, raw0);
  mask_past_vocab<kBf16>(zw, kc_of(0), a.vocab, lane);
  load_chunk<kBf16>(rows, loff, lstep, kc_of(2), raw0);

  // Group g: stage its embedding into slot g % 2 (every wave finished reading
  // that slot, group g - 2, before the barrier of group g - 1), put the next
  // group's loads in flight, and meet at the group's one barrier. Then each
  // wave runs the group's chunks on its own tile. Chunk j reads its operands,
  // then writes chunk j + 1 into the tile (a wave's LDS operations run in
  // order, so the reads see chunk j), reloads that chunk's register slot,
  // (j + 1) % 2, a constant since groups hold whole pairs, with chunk j + 3,
  // and multiplies.
  for (int32_t g = 0; g < ngroups; ++g) {
    uint16_t* eb = s_b[g & 1];
    stage_embed<kG>(eb, a, k_begin + static_cast<int64_t>(g) * kG * kScChunk, k_end, tid, ev);
    load_embed<kG>(a, kg_of(g + 1), k_end, voff, ev);
    __syncthreads();
    static_for<kG>([&](auto cc) {
      constexpr int ci = decltype(cc)::value;
      const int32_t j = g * kG + ci;
      // The older wave of each SIMD (waves 0-3) wins the issue arbiter and
      // would finish the group's chunks well before the younger one, then
      // wait at the next barrier while the younger runs alone; the younger
      // waves take the lead for the group's first half instead.
      if constexpr (ci == 0) {
        if (wave >= 4) __builtin_amdgcn_s_setprio(1);
      }
      if constexpr (ci == kG / 2) {
        if (wave >= 4) __builtin_amdgcn_s_setprio(0);
      }
      Operands o;
      read_operands(eb + ci * kEChunk, o);
      Raw<kBf16>& next = ci % 2 == 0 ? raw1 : raw0;
      store_chunk<kBf16>(zw, lane, next);
      mask_past_vocab<kBf16>(zw, kc_of(j + 1), a.vocab, lane);
      load_chunk<kBf16>(rows, loff, lstep, kc_of(j + 3), next);
      // (a chunk past the slice end, in its last group only, meets an all-zero
      // embedding tile and adds exactly zero; multiplying it anyway keeps the
      // group's code one block, so its reads are issued here)
      multiply(o);
    });
  }

  const f32x16_t acc = acc0 + acc1;
  // lane l, register r holds D[i][n] with n = l % 32 and
  // i = 8 (r / 4) + 4 (l / 32) + r % 4 (the 32x32 fp32 accumulator layout)
  const int n = lane & 31;
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
// One workgroup per row: thread t takes columns 4 (t % 8) .. +3 of the
// slices s = g, g + 32, g + 64, ... of group g = t / 8, all its loads in
// flight at once (rows of inactive canvases are read too and not written, so
// that no load waits for the flag). The 32 group sums are then combined in a
// fixed pattern (lanes 8, 16 and 32 apart within each wave, then the four
// waves in order), so the result does not depend on timing.
__global__ __launch_bounds__(256) void self_cond_reduce_kernel(SelfCondArgs a) {
  constexpr int kPerRound = 8;  // loads per thread and round: 256 slices in one round
  __shared__ float4 s_wave[4][8];
  const int32_t r = static_cast<int32_t>(blockIdx.x);
  const int t = threadIdx.x, quad = t & 7, group = t >> 3, lane = t & 63, wave = t >> 6;
  const int64_t stride = static_cast<int64_t>(a.rows_pad) * 32;
  const float* base = a.partials + static_cast<int64_t>(r) * 32 + 4 * quad;
  float4 sum = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int32_t s0 = group; s0 < a.nslice; s0 += 32 * kPerRound) {
    float4 v[kPerRound];
#pragma unroll
    for (int i = 0; i < kPerRound; ++i) {
      const int32_t sl = s0 + 32 * i;
      v[i] = *reinterpret_cast<const float4*>(base + (sl < a.nslice ? sl : a.nslice - 1) * stride);
    }
#pragma unroll
    for (int i = 0; i < kPerRound; ++i) {
      if (s0 + 32 * i < a.nslice) {
        sum.x += v[i].x;
        sum.y += v[i].y;
        sum.z += v[i].z;
        sum.w += v[i].w;
      }
    }
  }
#pragma unroll
  for (int m = 8; m < 64; m <<= 1) {
    sum.x += __shfl_xor(sum.x, m);
    sum.y += __shfl_xor(sum.y, m);
    sum.z += __shfl_xor(sum.z, m);
    sum.w += __shfl_xor(sum.w, m);
  }
  if (lane < 8) s_wave[wave][lane] = sum;
  __syncthreads();
  if (t < 32) {
    auto col = [&](int w, int k) {
      const float4 q = s_wave[w][k >> 2];
      const int e = k & 3;
      return e == 0 ? q.x : e == 1 ? q.y : e == 2 ? q.z : q.w;
    };
    const float tot = ((col(0, t) + col(1, t)) + col(2, t)) + col(3, t);
    const float den = ((col(0, a.d) + col(1, a.d)) + col(2, a.d)) + col(3, a.d);
    if (t < a.d && (a.active == nullptr || a.active[r / a.canvas_len] != 0))
      a.out[static_cast<int64_t>(r) * a.d + t] = tot / den;
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
