// lmhead_gemm_kernel: the LM-head projection that produces the logits the
// sampler consumes, logits[r, v] = sum_k hidden[r, k] * weight[k, v], with
// bf16 operands, fp32 accumulation on the matrix cores and fp32 logits.
// The pages' sampling stage is a full-vocabulary softmax over the 256 canvas
// positions ("DiffusionGemma: Parallel Denoising From an Autoregressive
// Checkpoint", the hardware breakdown); its logits come from this product.
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
//   * inside a wave tile, column n of MFMA tile t (n < 16, t < 8) is logit
//     column 8n + t, so each lane ends up holding 8 consecutive vocabulary
//     ids of every row it owns: one slot of the sampler's block geometry, and
//     one 32-byte store per row.
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

struct GemmLds {
  uint16_t a[2][kBM * kPitch];
  uint16_t b[2][kBN * kPitch];
};

__device__ __forceinline__ uint4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Low (hi_half = false) or high 16-bit halves of two words packed as (lo, hi).
__device__ __forceinline__ uint32_t pack_halves(uint32_t lo, uint32_t hi, bool hi_half) {
  return hi_half ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
}

__global__ __launch_bounds__(kGemmThreads, 1) void lmhead_gemm_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) GemmLds lds;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave >> 1;   // 0..3: rows wm * 64
  const int wn = wave & 1;    // 0..1: columns wn * 128

  const int32_t mtiles = (g.rows + kBM - 1) / kBM;
  const int32_t m0 = static_cast<int32_t>(blockIdx.x % static_cast<uint32_t>(mtiles)) * kBM;
  const int32_t n0 = static_cast<int32_t>(blockIdx.x / static_cast<uint32_t>(mtiles)) * kBN;
  const int32_t K = g.hidden_dim;
  const int32_t V = g.vocab;
  const int32_t nk = K / kBK;

  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(g.hidden), 0, g.rows * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(g.weight), 0, K * V * 2, 0x00020000);

  // hidden: thread loads rows (tid >> 3) + 64 j, k chunk tid & 7 (8 ids).
  // weight: thread loads k rows 4 * (tid >> 5) + j, columns 8 * (tid & 31) + [0, 8).
  // Rows past the last one and columns past V are clamped onto real data: the
  // products they feed land in rows and columns that are never stored, and
  // the loads stay unconditional (no branch, exact load-counter waits).
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
  const int32_t b_col = min(n0 + b_cg * 8, V - 8);
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
      *reinterpret_cast<uint4*>(&lds.a[buf][(a_row + 64 * j) * kPitch + a_kc * 8]) = ga[j];
    // transpose the 4 x 8 (k, v) block: column c of it becomes 4 k values of
    // logit column 8 * b_cg + c, stored at the LDS row of its MFMA tile
    const uint32_t* w = reinterpret_cast<const uint32_t*>(gb);  // w[4 j + i]: columns 2i, 2i+1 of k row j
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      uint2 col;
      col.x = pack_halves(w[0 * 4 + c / 2], w[1 * 4 + c / 2], c & 1);
      col.y = pack_halves(w[2 * 4 + c / 2], w[3 * 4 + c / 2], c & 1);
      const int r = (b_cg >> 4) * 128 + c * 16 + (b_cg & 15);
      *reinterpret_cast<uint2*>(&lds.b[buf][r * kPitch + b_kq * 4]) = col;
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
            &lds.a[cur][(wm * 64 + i * 16 + frag_row) * kPitch + kk * 32 + frag_k]);
#pragma unroll
      for (int t = 0; t < 8; ++t)
        bfr[t] = *reinterpret_cast<const bf16x8_t*>(
            &lds.b[cur][(wn * 128 + t * 16 + frag_row) * kPitch + kk * 32 + frag_k]);
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

  // lane holds rows 4 * (lane >> 4) + [0, 4) of each MFMA tile and columns
  // 8 * (lane & 15) + t of the wave tile
  const int32_t col = n0 + wn * 128 + 8 * (lane & 15);
  if (col >= V) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int32_t row = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + q;
      if (row < g.rows) {
        float* dst = g.logits + static_cast<int64_t>(row) * g.ld_logits + col;
        reinterpret_cast<float4*>(dst)[0] = make_float4(acc[i][0][q], acc[i][1][q], acc[i][2][q], acc[i][3][q]);
        reinterpret_cast<float4*>(dst)[1] = make_float4(acc[i][4][q], acc[i][5][q], acc[i][6][q], acc[i][7][q]);
      }
    }
  }
}

}  // namespace

hipError_t launch_lmhead_gemm(const GemmArgs& g, hipStream_t stream) {
  const uint32_t mtiles = static_cast<uint32_t>((g.rows + kBM - 1) / kBM);
  const uint32_t ntiles = static_cast<uint32_t>((g.vocab + kBN - 1) / kBN);
  hipLaunchKernelGGL(lmhead_gemm_kernel, dim3(mtiles * ntiles), dim3(kGemmThreads), 0, stream, g);
  return hipGetLastError();
}

}  // namespace dg
