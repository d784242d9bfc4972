// The self-conditioning matmul of the sampling stage: for each row r (a canvas
// position) the expected token embedding under the step's tempered prediction,
//   out[r, n] = sum_v p_r(v) E[v, n],  p_r = softmax(z_r / T),
// in fp32 ("DiffusionGemma: Parallel Denoising From an Autoregressive
// Checkpoint", "Finding": the self-conditioning block feeds the previous
// prediction back; hardware paragraph: the sampling stage runs it with the
// full-vocabulary softmax, in full precision, over the canvas positions).
//
// It is a contraction over the vocabulary (K = V, M = rows, N = d + 1 with the
// normaliser), so it runs on the fp32 matrix cores (v_mfma_f32_32x32x2f32):
//   - a workgroup owns 256 rows (8 waves x 32) and a slice of the vocabulary;
//   - per 64-id chunk, lane l of a wave loads 32 consecutive logits of row
//     l % 32 (ids +0..31 for l < 32, +32..63 for l >= 32: the two halves read
//     one 128-byte line of the row together) and turns them into
//     e = 2^(z c - zmax c), c = log2(e)/T, with zmax the row's largest logit
//     (read at the argmax the statistics pass found), so e <= 1;
//   - the chunk's 64 embedding rows are staged in LDS as 32 columns: E[v, 0..d-1],
//     a column of ones at d (its sum is the normaliser S = sum_v e_v) and zeros
//     above; MFMA j multiplies lane values e_j (ids j and 32 + j of the chunk)
//     with the matching LDS rows;
//   - one slice per row tile: the workgroup divides by S and writes out;
//     otherwise it writes its unnormalised partial tile, and a second kernel
//     sums the slices in a fixed order and divides.
#include "device_common.h"
#include "kernels.h"

namespace dg {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2eSc = 1.4426950408889634f;
constexpr int kScChunk = 64;

template <bool kBf16>
__device__ __forceinline__ float logit_at(const void* base, int64_t i) {
  if constexpr (kBf16) {
    const uint16_t b = static_cast<const uint16_t*>(base)[i];
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
  } else {
    return static_cast<const float*>(base)[i];
  }
}

// The 32 logits of ids id0 .. id0+31 of one row (id0 a multiple of 32), zero
// past `end`. 16-byte pieces never cross the row's padded end: the row stride
// is a multiple of 16 bytes and every piece starts below `end` <= V.
template <bool kBf16>
__device__ __forceinline__ void load32(const void* row_base, int64_t id0, int64_t end, float (&z)[32]) {
  constexpr int kPer = kBf16 ? 8 : 4;
#pragma unroll
  for (int q = 0; q < 32 / kPer; ++q) {
    const int64_t id = id0 + q * kPer;
    uint4 w = make_uint4(0u, 0u, 0u, 0u);
    if (id < end) {
      if constexpr (kBf16)
        w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(row_base) + id);
      else
        w = *reinterpret_cast<const uint4*>(static_cast<const float*>(row_base) + id);
    }
    if constexpr (kBf16) {
      const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        z[q * 8 + 2 * h] = __uint_as_float(u[h] << 16);
        z[q * 8 + 2 * h + 1] = __uint_as_float(u[h] & 0xFFFF0000u);
      }
    } else {
      z[q * 4 + 0] = __uint_as_float(w.x);
      z[q * 4 + 1] = __uint_as_float(w.y);
      z[q * 4 + 2] = __uint_as_float(w.z);
      z[q * 4 + 3] = __uint_as_float(w.w);
    }
  }
}

// The chunk's embedding rows as this thread stages them: elements
// kScStage t .. kScStage t + kScStage - 1 of the [64][32] tile (row = element
// / 32, column = element % 32).
constexpr int kScStage = kScChunk * 32 / kScThreads;

__device__ __forceinline__ void load_embed(const SelfCondArgs& a, int64_t kc, int64_t k_end, int tid,
                                           float (&ev)[kScStage]) {
#pragma unroll
  for (int q = 0; q < kScStage; ++q) {
    const int idx = tid * kScStage + q, n = idx & 31;
    const int64_t v = kc + (idx >> 5);
    float e = 0.0f;
    if (v < k_end) e = n < a.d ? a.embed[v * a.d + n] : (n == a.d ? 1.0f : 0.0f);
    ev[q] = e;
  }
}

template <bool kBf16>
__global__ __launch_bounds__(kScThreads) void self_cond_kernel(SelfCondArgs a) {
  __shared__ float s_e[2][kScChunk][32];
  const int32_t tile = static_cast<int32_t>(blockIdx.x) / a.nslice;
  const int32_t slice = static_cast<int32_t>(blockIdx.x) % a.nslice;
  const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int32_t row = tile * kScRowTile + wave * 32 + (lane & 31);
  const bool row_ok = row < a.rows;

  float c = 0.0f, mc = 0.0f;
  const void* row_base = a.logits;
  if (row_ok) {
    const int64_t off = static_cast<int64_t>(row) * a.row_stride;
    row_base = kBf16 ? static_cast<const void*>(static_cast<const uint16_t*>(a.logits) + off)
                     : static_cast<const void*>(static_cast<const float*>(a.logits) + off);
    int32_t am = a.argmax[row];
    am = am < 0 ? 0 : (am >= a.vocab ? a.vocab - 1 : am);
    c = kLog2eSc / a.temperature[row / a.canvas_len];
    mc = logit_at<kBf16>(row_base, am) * c;
  }
  const int64_t k_begin = static_cast<int64_t>(slice) * a.kslice;
  const int64_t k_end = k_begin + a.kslice < a.vocab ? k_begin + a.kslice : a.vocab;
  const int64_t row_end = row_ok ? k_end : 0;  // rows past the batch contribute nothing

  // software pipeline: the loads of chunk i + 1 are in flight while chunk i
  // is turned into probabilities and multiplied; the embedding tile is
  // double-buffered in LDS, so one barrier per chunk suffices
  float z[32], ev[kScStage];
  load32<kBf16>(row_base, k_begin + 32 * half, row_end, z);
  load_embed(a, k_begin, k_end, tid, ev);
  f32x16_t acc0 = {}, acc1 = {};
  int buf = 0;
  for (int64_t kc = k_begin; kc < k_end; kc += kScChunk, buf ^= 1) {
#pragma unroll
    for (int q = 0; q < kScStage; ++q) {
      const int idx = tid * kScStage + q;
      s_e[buf][idx >> 5][idx & 31] = ev[q];
    }
    float p[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const int64_t id = kc + 32 * half + j;
      p[j] = id < row_end ? __builtin_amdgcn_exp2f(__builtin_fmaf(z[j], c, -mc)) : 0.0f;
    }
    const int64_t kn = kc + kScChunk;
    if (kn < k_end) {
      load32<kBf16>(row_base, kn + 32 * half, row_end, z);
      load_embed(a, kn, k_end, tid, ev);
    }
    __syncthreads();  // this chunk's embedding rows are in LDS; the other buffer is free again
#pragma unroll
    for (int j = 0; j < 32; j += 2) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(p[j], s_e[buf][j + 32 * half][lane & 31], acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(p[j + 1], s_e[buf][j + 1 + 32 * half][lane & 31], acc1, 0,
                                                  0, 0);
    }
  }
  const f32x16_t acc = acc0 + acc1;
  // lane l, register r holds D[i][n] with n = l % 32 and
  // i = 8 (r / 4) + 4 (l / 32) + r % 4 (the 32x32 fp32 accumulator layout)
  const int n = lane & 31;
  const int32_t row0 = tile * kScRowTile + wave * 32;
  if (a.nslice == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float s = __shfl(acc[r], (lane & 32) | a.d);  // the normaliser of this row
      const int32_t gr = row0 + 8 * (r >> 2) + 4 * half + (r & 3);
      if (gr < a.rows && n < a.d) a.out[static_cast<int64_t>(gr) * a.d + n] = acc[r] / s;
    }
  } else {
    float* part = a.partials + static_cast<int64_t>(slice) * a.rows_pad * 32;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int32_t gr = row0 + 8 * (r >> 2) + 4 * half + (r & 3);
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
