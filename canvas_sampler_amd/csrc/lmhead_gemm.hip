// lmhead_gemm_kernel: the LM-head projection that produces the logits the
// sampler consumes, logits[r, v] = sum_k hidden[r, k] * weight[k, v], with
// bf16 operands and fp32 accumulation on the matrix cores. The pages'
// sampling stage is a full-vocabulary softmax over the 256 canvas positions
// ("DiffusionGemma: Parallel Denoising From an Autoregressive Checkpoint",
// the hardware breakdown); its logits come from this product.
//
// Two epilogues share one main loop, so both see the same fp32 logits bit
// for bit:
//   * store: the tile's logits are written out (fp32);
//   * statistics: the logits never leave the chip. A tile's 256 columns are
//     chosen to be four whole blocks of the sampler's two-level Gumbel-max
//     protocol (block j = one 8-id slot across the eight 512-id stripes of a
//     4096-id chunk), and for each of its 256 rows the tile reduces them to
//     one 40-byte partial: max logit and its first id, the sums of 2^t and
//     t * 2^t (t = z log2(e) / T - ref) that give the entropy, and the best of
//     its four block scores (log2-sum-exp plus the block's Gumbel) with the
//     in-block Gumbel-max draw of that block. A per-row running best score
//     (atomic maximum) lets tiles whose best block is already beaten skip the
//     draw; the row's partials are merged afterwards by partials_merge_kernel.
//
// Tiling (gfx950, wave64, v_mfma_f32_16x16x32_bf16):
//   * a workgroup of 8 waves computes a 256 x 256 tile of logits; the waves
//     form a 4 x 2 grid of 64 x 128 wave tiles, i.e. 4 x 8 MFMA tiles of
//     16 x 16 held in 128 fp32 accumulators per lane (two waves per SIMD,
//     everything in the 256 architectural registers of each);
//   * K advances 64 at a time through two LDS stages (144 KiB): while the
//     matrix cores work on one stage, the next stage is written to the other
//     from registers and the loads of the stage after it are in flight;
//   * hidden is K-contiguous, so its 16-byte loads go to LDS unchanged;
//     weight is V-contiguous, so each lane loads a 4 x 8 (k, v) block and
//     transposes it in registers, giving K-contiguous LDS rows from which
//     every MFMA operand is one 16-byte LDS read;
//   * inside a wave tile, column n of MFMA tile t (n < 16, t < 8) is tile
//     column 8n + t, so each lane ends up holding one 8-column piece of every
//     row it owns. With the store epilogue piece p of a tile is columns
//     n0 + 8p + [0, 8) (one 32-byte store per row); with the statistics
//     epilogue it is stripe p / 4 of slot 4 qb + p % 4 of the tile's chunk, so
//     a lane holds one eighth of a block and the four lanes of a DPP row with
//     the same p % 4 hold half of it (the other wave of the pair the rest).
// LDS rows are padded to 144 bytes so that the 16-byte operand reads of a
// wave are free of bank conflicts.

#include "device_common.h"
#include "kernels.h"

namespace dg {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kBK = 64;
constexpr int kPitch = kBK + 8;          // bf16 elements per LDS row (144 bytes)
constexpr int kTilesPerChunk = kChunkIds / kBN;   // 16: four blocks per tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

constexpr int kBlkPitch = 68;   // floats per parked block row (64 logits, padded)

struct GemmLds {
  uint16_t a[2][kBM * kPitch];
  uint16_t b[2][kBN * kPitch];
};

// Per-row exchange area of the statistics epilogue (after the main loop the
// operand stages are dead and this overlays them). "Half" is the wave column
// wn: stripes 0-3 (wn = 0) or 4-7 (wn = 1) of each block.
struct EpiLds {
  float c[kBM];            // log2(e) / T of each local row
  float inv_t[kBM];        // 1 / T
  int32_t pos[kBM];        // canvas position (counter word 1)
  int32_t step[kBM];       // counter word 2
  uint32_t k0[kBM];        // Philox key: the canvas seed
  uint32_t k1[kBM];
  uint32_t hint[kBM];      // the row's best block score seen when the tile started
  float hmax[2][kBM];      // largest logit of each half
  int32_t hkey[2][kBM];    // its first position key (s * 32 + u * 8 + t), or INT_MAX
  float hs[2][kBM][4];     // half-block sums of 2^t
  float hw[2][kBM][4];     // half-block sums of t * 2^t
  int32_t draw_u[kBM];     // block (0..3) to draw in, or -1
  int32_t sample[kBM];     // the draw's id
  float blk[kBM][kBlkPitch];  // the 64 logits of each drawn block (-inf past V), by stripe and id
  RowPartial fin[kBM];
};

static_assert(sizeof(EpiLds) <= sizeof(GemmLds), "the epilogue's LDS overlays the operand stages");

union TileLds {
  GemmLds g;
  EpiLds e;
};

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Low (hi_half = false) or high 16-bit halves of two words packed as (lo, hi).
__device__ __forceinline__ uint32_t pack_halves(uint32_t lo, uint32_t hi, bool hi_half) {
  return hi_half ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
}

// Cross-lane moves inside a DPP row of 16 lanes for the reductions of the
// statistics epilogue (every control used here has an in-row source for every
// lane, so no lane keeps an old value).
template <int C>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), C, 0xF, 0xF, true));
}

template <int C>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_mov_dpp(v, C, 0xF, 0xF, true);
}

__device__ __forceinline__ uint64_t row16_max_u64(uint64_t k) {
  k = max_u64(k, dpp_mov_u64<kDppXor8>(k));
  k = max_u64(k, dpp_mov_u64<kDppRor4>(k));
  k = max_u64(k, dpp_mov_u64<kDppXor2>(k));
  return max_u64(k, dpp_mov_u64<kDppXor1>(k));
}

__device__ __forceinline__ uint32_t word_of(const Words4& w, int k) {
  return k == 0 ? w.w[0] : k == 1 ? w.w[1] : k == 2 ? w.w[2] : w.w[3];
}

// Order-preserving bits of a score (never NaN): a larger score has larger bits,
// and every score lies above 0.
__device__ __forceinline__ uint32_t ordered_bits(float x) {
  const uint32_t b = x == 0.0f ? 0u : __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <bool kStats>
__global__ __launch_bounds__(kGemmThreads, 1) void lmhead_gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) TileLds lds;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave >> 1;   // 0..3: rows wm * 64
  const int wn = wave & 1;    // 0..1: columns wn * 128

  const int32_t mtiles = (g.rows + kBM - 1) / kBM;
  const int32_t mt = static_cast<int32_t>(blockIdx.x % static_cast<uint32_t>(mtiles));
  const int32_t nt = static_cast<int32_t>(blockIdx.x / static_cast<uint32_t>(mtiles));
  const int32_t m0 = mt * kBM;
  const int32_t K = g.hidden_dim;
  const int32_t V = g.vocab;
  const int32_t nk = K / kBK;
  // statistics epilogue: the tile is quarter qb of chunk ch (slots 4 qb .. 4 qb + 3)
  const int32_t ch = nt / kTilesPerChunk;
  const int32_t qb = nt % kTilesPerChunk;
  // first vocabulary id of tile piece p (8 consecutive ids)
  auto piece_id = [&](int p) -> int32_t {
    if constexpr (kStats)
      return ch * kChunkIds + (p >> 2) * kStripeIds + (4 * qb + (p & 3)) * kSlotIds;
    else
      return nt * kBN + p * 8;
  };

  // per-canvas values of local row tid (threads 0..255), fetched before the
  // main loop and parked in LDS after it
  float rc_temp = 1.0f;
  int32_t rc_step = 0, rc_pos = 0;
  uint64_t rc_seed = 0;
  if constexpr (kStats) {
    if (g.active != nullptr) {
      // a tile whose rows all belong to inactive canvases has nothing to do
      const int32_t c_first = m0 / g.canvas_len;
      const int32_t c_last = (min(m0 + kBM, g.rows) - 1) / g.canvas_len;
      bool any = false;
      for (int32_t c = c_first; c <= c_last; ++c) any = any || g.active[c] != 0;
      if (!any) return;
    }
    if (tid < kBM) {
      const int32_t row = min(m0 + tid, g.rows - 1);
      const int32_t canvas = row / g.canvas_len;
      rc_pos = row - canvas * g.canvas_len;
      rc_temp = g.temperature[canvas];
      rc_step = g.steps != nullptr ? g.steps[canvas] : g.step;
      rc_seed = g.seeds[canvas];
    }
  }

  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(g.hidden), 0, g.rows * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(g.weight), 0, K * V * 2, 0x00020000);

  // hidden: thread loads rows (tid >> 3) + 64 j, k chunk tid & 7 (8 ids).
  // weight: thread loads k rows 4 * (tid >> 5) + j, the 8 columns of piece
  // tid & 31. Rows past the last one and columns past V are clamped onto real
  // data: the products they feed land in rows and columns that are never
  // used, and the loads stay unconditional (no branch, exact load-counter
  // waits).
  const int a_row = tid >> 3;
  const int a_kc = tid & 7;
  const int b_kq = tid >> 5;
  const int b_cg = tid & 31;
  uint32_t a_base[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int32_t row = min(m0 + a_row + 64 * j, g.rows - 1);
    a_base[j] = static_cast<uint32_t>((row * K + a_kc * 8) * 2);
  }
  const int32_t b_col = min(piece_id(b_cg), V - 8);
  const uint32_t b_base = static_cast<uint32_t>((b_kq * 4 * V + b_col) * 2);
  const uint32_t b_krow = static_cast<uint32_t>(V * 2);

  uint4 ga[4];
  uint4 gb[4];
  // stage kt of K (the prefetch past the last stage reloads the last one)
  auto load_stage = [&](int kt) {
    const int32_t ks = min(kt, nk - 1);
#pragma unroll
    for (int j = 0; j < 4; ++j) ga[j] = load16(ra, a_base[j] + static_cast<uint32_t>(ks * kBK * 2));
    const uint32_t boff = b_base + static_cast<uint32_t>(ks * kBK) * b_krow;
#pragma unroll
    for (int j = 0; j < 4; ++j) gb[j] = load16(rb, boff + static_cast<uint32_t>(j) * b_krow);
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<uint4*>(&lds.g.a[buf][(a_row + 64 * j) * kPitch + a_kc * 8]) = ga[j];
    // transpose the 4 x 8 (k, v) block: column c of it becomes 4 k values of
    // tile column 8 * b_cg + c, stored at the LDS row of its MFMA tile
    const uint32_t* w = reinterpret_cast<const uint32_t*>(gb);  // w[4 j + i]: columns 2i, 2i+1 of k row j
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint2 col;
      col.x = pack_halves(w[0 * 4 + c / 2], w[1 * 4 + c / 2], c & 1);
      col.y = pack_halves(w[2 * 4 + c / 2], w[3 * 4 + c / 2], c & 1);
      const int r = (b_cg >> 4) * 128 + c * 16 + (b_cg & 15);
      *reinterpret_cast<uint2*>(&lds.g.b[buf][r * kPitch + b_kq * 4]) = col;
    }
  };

  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[i][t] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Stage kt + 1 is written to LDS in the middle of iteration kt, between the
  // two K halves of stage kt, from registers loaded one iteration before; the
  // loads of stage kt + 2 go out right after. The writes then overlap the
  // matrix cores instead of stalling every wave at the top of the iteration
  // (the written buffer is read only after the barrier that ends kt). The
  // MFMA groups run at raised issue priority.
  load_stage(0);
  store_stage(0);
  load_stage(1);
  __syncthreads();

  const int frag_row = lane & 15;
  const int frag_k = 8 * (lane >> 4);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
#pragma unroll
    for (int kk = 0; kk < kBK / 32; ++kk) {
      if (kk == 1) {
        store_stage(cur ^ 1);
        load_stage(kt + 2);
      }
      bf16x8_t af[4];
      bf16x8_t bfr[8];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(
            &lds.g.a[cur][(wm * 64 + i * 16 + frag_row) * kPitch + kk * 32 + frag_k]);
#pragma unroll
      for (int t = 0; t < 8; ++t)
        bfr[t] = *reinterpret_cast<const bf16x8_t*>(
            &lds.g.b[cur][(wn * 128 + t * 16 + frag_row) * kPitch + kk * 32 + frag_k]);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[t], acc[i][t], 0, 0, 0);
      __builtin_amdgcn_s_setprio(0);
    }
    __syncthreads();
  }

  // lane holds rows 4 * (lane >> 4) + [0, 4) of each MFMA tile and the 8
  // columns of piece 16 wn + (lane & 15)
  const int n = lane & 15;
  const int32_t id0 = piece_id(wn * 16 + n);
  if constexpr (!kStats) {
    if (id0 >= V) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int32_t row = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + q;
        if (row < g.rows) {
          float* dst = g.logits + static_cast<int64_t>(row) * g.ld_logits + id0;
          reinterpret_cast<float4*>(dst)[0] = make_float4(acc[i][0][q], acc[i][1][q], acc[i][2][q], acc[i][3][q]);
          reinterpret_cast<float4*>(dst)[1] = make_float4(acc[i][4][q], acc[i][5][q], acc[i][6][q], acc[i][7][q]);
        }
      }
    }
  } else {
    // ---- statistics epilogue. u = block of the lane's piece (0..3), stripe
    // s = 4 wn + (n >> 2). Local order key of id t of the piece: s * 32 +
    // u * 8 + t, which increases with the id.
    EpiLds& e = lds.e;
    const int u = n & 3;
    const bool ok = id0 < V;   // V is a multiple of 8: whole pieces are in or out
    const int key0 = (4 * wn + (n >> 2)) * 32 + u * 8;
    auto local_row = [&](int i, int q) { return wm * 64 + i * 16 + 4 * (lane >> 4) + q; };

    if (tid < kBM) {
      e.c[tid] = kLog2e / rc_temp;
      e.inv_t[tid] = 1.0f / rc_temp;
      e.pos[tid] = rc_pos;
      e.step[tid] = rc_step;
      e.k0[tid] = static_cast<uint32_t>(rc_seed);
      e.k1[tid] = static_cast<uint32_t>(rc_seed >> 32);
    }
    // the row's running best block score, read now (its latency hides behind
    // phases 1 and 2) and parked for phase 3
    uint32_t rc_hint = 0;
    if (tid < kBM)
      rc_hint = __hip_atomic_load(&g.hint[min(m0 + tid, g.rows - 1)], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // phase 1: largest logit of each half row. The reductions over a DPP
    // row run step by step across all 16 row slots, so that consecutive
    // cross-lane moves are independent.
    {
      float m[16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float v = max3_raw(max3_raw(acc[i][0][q], acc[i][1][q], acc[i][2][q]),
                                   max3_raw(acc[i][3][q], acc[i][4][q], acc[i][5][q]),
                                   max_raw(acc[i][6][q], acc[i][7][q]));
          m[4 * i + q] = ok ? v : kNegInf;
        }
#pragma unroll
      for (int r = 0; r < 16; ++r) m[r] = max_raw(m[r], dpp_f<kDppXor8>(m[r]));
#pragma unroll
      for (int r = 0; r < 16; ++r) m[r] = max_raw(m[r], dpp_f<kDppRor4>(m[r]));
#pragma unroll
      for (int r = 0; r < 16; ++r) m[r] = max_raw(m[r], dpp_f<kDppXor2>(m[r]));
#pragma unroll
      for (int r = 0; r < 16; ++r) m[r] = max_raw(m[r], dpp_f<kDppXor1>(m[r]));
      if (n == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) e.hmax[wn][local_row(r >> 2, r & 3)] = m[r];
      }
    }
    __syncthreads();

    // phase 2: against ref = tile max * c, the half-block sums and the first
    // position of the tile maximum (reductions batched as in phase 1)
    {
      float sv[16], wv[16];
      int kv[16];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int lr = local_row(i, q);
          const float tm = max_raw(e.hmax[0][lr], e.hmax[1][lr]);
          const float c = e.c[lr];
          const float ref = __fmul_rn(tm, c);
          float ex[8];
          float w4[4] = {0.f, 0.f, 0.f, 0.f};
          int kf = 8;
#pragma unroll
          for (int t = 7; t >= 0; --t) kf = acc[i][t][q] == tm ? t : kf;
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const float tt = fmaf(acc[i][t][q], c, -ref);
            ex[t] = __builtin_amdgcn_exp2f(tt);
            w4[t & 3] = fmaf(tt, ex[t], w4[t & 3]);
          }
          const float s = ((ex[0] + ex[1]) + (ex[2] + ex[3])) + ((ex[4] + ex[5]) + (ex[6] + ex[7]));
          const float w = (w4[0] + w4[1]) + (w4[2] + w4[3]);
          sv[4 * i + q] = ok ? s : 0.0f;
          wv[4 * i + q] = ok ? w : 0.0f;
          kv[4 * i + q] = ok && kf < 8 ? key0 + kf : 0x7FFFFFFF;
        }
      // half-block sums over lanes n, n ^ 4, n ^ 8, n ^ 12 (lane i adds lane
      // i ^ 8, then lane (i - 4) mod 16: the same bits in all four), and the
      // first position over the row's 16 lanes
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sv[r] += dpp_f<kDppXor8>(sv[r]);
        wv[r] += dpp_f<kDppXor8>(wv[r]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sv[r] += dpp_f<kDppRor4>(sv[r]);
        wv[r] += dpp_f<kDppRor4>(wv[r]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) kv[r] = min(kv[r], dpp_i<kDppXor8>(kv[r]));
#pragma unroll
      for (int r = 0; r < 16; ++r) kv[r] = min(kv[r], dpp_i<kDppRor4>(kv[r]));
#pragma unroll
      for (int r = 0; r < 16; ++r) kv[r] = min(kv[r], dpp_i<kDppXor2>(kv[r]));
#pragma unroll
      for (int r = 0; r < 16; ++r) kv[r] = min(kv[r], dpp_i<kDppXor1>(kv[r]));
      if (n < 4) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int lr = local_row(r >> 2, r & 3);
          e.hs[wn][lr][n] = sv[r];
          e.hw[wn][lr][n] = wv[r];
        }
      }
      if (n == 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) e.hkey[wn][local_row(r >> 2, r & 3)] = kv[r];
      }
      if (tid < kBM) e.hint[tid] = rc_hint;
    }
    __syncthreads();

    // phase 3: thread t takes blocks 2 (t & 1) + {0, 1} of local row t >> 1
    // (its partner lane t ^ 1 the other two): their Gumbels (the Philox call
    // of block j is at counter j with bits 9-10 cleared, word (j >> 9) & 3),
    // sums and scores, then over the pair the tile's best block, its sums in
    // fp64, the first id of its maximum, and whether to draw
    {
      const int lr = tid >> 1;
      const int ub = 2 * (tid & 1);
      const float tm = max_raw(e.hmax[0][lr], e.hmax[1][lr]);
      const float ref = __fmul_rn(tm, e.c[lr]);
      const uint32_t pos = static_cast<uint32_t>(e.pos[lr]), stp = static_cast<uint32_t>(e.step[lr]);
      const uint32_t k0 = e.k0[lr], k1 = e.k1[lr];
      uint64_t kb = 0;
      double s = 0.0, w = 0.0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int ub2 = ub + h;
        const uint32_t j = static_cast<uint32_t>(ch * kSlots + 4 * qb + ub2);
        const Words4 wd = philox4x32_10(j & ~0x600u, pos, stp, kTagBlock, k0, k1);
        const float g2 = kLog2e * gumbel(word_of(wd, static_cast<int>((j >> 9) & 3)));
        const float sb = e.hs[0][lr][ub2] + e.hs[1][lr][ub2];
        const float wb = e.hw[0][lr][ub2] + e.hw[1][lr][ub2];
        const float score = sb > 0.0f ? ref + __log2f(sb) + g2 : kNegInf;
        kb = max_u64(kb, argmax_key(score, ub2));
        s += static_cast<double>(sb);
        w += static_cast<double>(wb);
      }
      kb = max_u64(kb, dpp_mov_u64<kDppXor1>(kb));
      s += dpp_mov_f64<kDppXor1>(s);
      w += dpp_mov_f64<kDppXor1>(w);
      if ((tid & 1) == 0) {
        float best;
        int ubest;
        argmax_unkey(kb, best, ubest);
        const int key = min(e.hkey[0][lr], e.hkey[1][lr]);
        RowPartial f;
        f.s = s;
        f.w = w;
        f.ref = tm == kNegInf ? kNegInf : ref;
        f.m = tm;
        f.argmax = key == 0x7FFFFFFF ? 0x7FFFFFFF
                                     : ch * kChunkIds + (key >> 5) * kStripeIds +
                                           (4 * qb + ((key >> 3) & 3)) * kSlotIds + (key & 7);
        const bool has = best != kNegInf;
        f.best = best;
        f.bestj = has ? ch * kSlots + 4 * qb + ubest : 0x7FFFFFFF;
        f.sample = 0x7FFFFFFF;
        // draw unless an earlier tile's best block of this row beats this
        // one's strictly: the row's best block then always draws
        const uint32_t ob = ordered_bits(best);
        const bool draw = has && ob >= e.hint[lr];
        const int32_t row = m0 + lr;
        if (draw && row < g.rows)
          __hip_atomic_fetch_max(&g.hint[row], ob, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        e.draw_u[lr] = draw ? ubest : -1;
        e.fin[lr] = f;
      }
    }
    __syncthreads();

    // phase 4: the in-block draws, argmax of z/T + G over the block's 64 ids
    // (lowest id on ties), G from the Philox call at counter id >> 2, word
    // id & 3. The lanes holding a drawn block park its logits in LDS; then
    // each DPP row of 16 lanes takes one drawing row, a lane per 4 ids (one
    // Philox call), so that the work scales with the number of draws.
    // the draw decisions of the lane's 16 row slots, read at once (draws are
    // rare, and one read per slot in the loop would wait on each in turn)
    int udv[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) udv[r] = e.draw_u[local_row(r >> 2, r & 3)];
    bool any_draw = false;
#pragma unroll
    for (int r = 0; r < 16; ++r) any_draw = any_draw || udv[r] >= 0;
    if (__builtin_amdgcn_ballot_w64(any_draw) != 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int lr = local_row(i, q);
        const int ud = udv[4 * i + q];
        if (__builtin_amdgcn_ballot_w64(ud >= 0) == 0) continue;
        if (ud == u) {
          float* dst = &e.blk[lr][(4 * wn + (n >> 2)) * kSlotIds];
          reinterpret_cast<float4*>(dst)[0] = ok ? make_float4(acc[i][0][q], acc[i][1][q], acc[i][2][q], acc[i][3][q])
                                                 : make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
          reinterpret_cast<float4*>(dst)[1] = ok ? make_float4(acc[i][4][q], acc[i][5][q], acc[i][6][q], acc[i][7][q])
                                                 : make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
        }
      }
    }
    __syncthreads();
    {
      const int quad = tid & 15;   // ids 4 quad .. 4 quad + 3 of the block: stripe quad / 2
      constexpr int kIters = kBM / (kGemmThreads / 16);
      int udr[kIters];
#pragma unroll
      for (int it = 0; it < kIters; ++it) udr[it] = e.draw_u[it * (kGemmThreads / 16) + (tid >> 4)];
#pragma unroll
      for (int it = 0; it < kIters; ++it) {
        const int lr = it * (kGemmThreads / 16) + (tid >> 4);
        const int ud = udr[it];
        if (__builtin_amdgcn_ballot_w64(ud >= 0) == 0) continue;
        float sc = kNegInf;
        int32_t id = 0x7FFFFFFF;
        if (ud >= 0) {
          const int32_t q0 = ch * kChunkIds + (quad >> 1) * kStripeIds + (4 * qb + ud) * kSlotIds + 4 * (quad & 1);
          const Words4 wd = philox4x32_10(static_cast<uint32_t>(q0 >> 2), static_cast<uint32_t>(e.pos[lr]),
                                          static_cast<uint32_t>(e.step[lr]), kTagElem, e.k0[lr], e.k1[lr]);
          const float4 z = reinterpret_cast<const float4*>(&e.blk[lr][4 * quad])[0];
          const float inv_t = e.inv_t[lr];
          const float zz[4] = {z.x, z.y, z.z, z.w};
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float v = zz[t] * inv_t + gumbel(wd.w[t]);
            if (v > sc) {
              sc = v;
              id = q0 + t;
            }
          }
        }
        const uint64_t k = row16_max_u64(argmax_key(sc, id));
        if (quad == 0 && ud >= 0) {
          float best;
          int32_t smp;
          argmax_unkey(k, best, smp);
          e.sample[lr] = smp;
        }
      }
    }
    __syncthreads();

    // phase 5: threads 0..255 write the partials of their local rows
    if (tid < kBM) {
      const int32_t row = m0 + tid;
      if (row < g.rows) {
        RowPartial f = e.fin[tid];
        if (e.draw_u[tid] >= 0) f.sample = e.sample[tid];
        g.partials[static_cast<int64_t>(row) * g.ntiles + nt] = f;
      }
    }
  }
}

}  // namespace

hipError_t launch_lmhead_gemm(const GemmArgs& g, hipStream_t stream) {
  const uint32_t mtiles = static_cast<uint32_t>((g.rows + kBM - 1) / kBM);
  const uint32_t ntiles = static_cast<uint32_t>((g.vocab + kBN - 1) / kBN);
  hipLaunchKernelGGL(lmhead_gemm_kernel<false>, dim3(mtiles * ntiles), dim3(kGemmThreads), 0, stream, g);
  return hipGetLastError();
}

int32_t lmhead_stats_tiles(int32_t vocab) { return ((vocab + kChunkIds - 1) / kChunkIds) * kTilesPerChunk; }

hipError_t launch_lmhead_stats(const GemmArgs& g, hipStream_t stream) {
  const uint32_t mtiles = static_cast<uint32_t>((g.rows + kBM - 1) / kBM);
  const uint32_t ntiles = static_cast<uint32_t>(g.ntiles);
  hipError_t err = launch_fill_u32(g.hint, g.rows, 0u, stream);
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(lmhead_gemm_kernel<true>, dim3(mtiles * ntiles), dim3(kGemmThreads), 0, stream, g);
  return hipGetLastError();
}

}  // namespace dg
