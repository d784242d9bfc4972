// accept_renoise_kernel and canvas_init_kernel: the per-canvas decisions of a
// sampler step (accept_canvas, one workgroup per canvas) and the initial canvas.

#include "accept_core.h"
#include "device_common.h"
#include "kernels.h"

namespace dg {
namespace {

__global__ __launch_bounds__(kAcceptThreads) void accept_renoise_kernel(AcceptArgs a) {
  const int32_t canvas = blockIdx.x;
  // every load goes out before the first is used (the active flag included:
  // an inactive canvas's inputs are valid memory, only unused)
  const AcceptInputs in = load_accept_inputs(a, canvas, threadIdx.x);
  if (a.active != nullptr && a.active[canvas] == 0) return;
  accept_canvas<kAcceptThreads>(a, canvas, in);
}

// Initial canvas: position l of canvas c gets floor(w0 * V / 2^32) with w0
// from Philox(seed_c; (0, l, 0, INIT)) ("DiffusionGemma Lab", §2 item 1).
__global__ void canvas_init_kernel(const uint64_t* __restrict__ seeds, int32_t canvas_len,
                                   int32_t vocab, int64_t total, int32_t* __restrict__ canvas) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int32_t c = static_cast<int32_t>(i / canvas_len);
  const int32_t l = static_cast<int32_t>(i % canvas_len);
  const uint64_t seed = seeds[c];
  const Words4 rw = philox4x32_10(0u, static_cast<uint32_t>(l), 0u, kTagInit,
                                  static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32));
  canvas[i] = uniform_token(rw.w[0], static_cast<uint32_t>(vocab));
}

__global__ void run_state_init_kernel(int32_t batch, uint8_t* __restrict__ active,
                                      int32_t* __restrict__ steps_used, uint8_t* __restrict__ stopped,
                                      float* __restrict__ temperature, float t0) {
  const int32_t c = static_cast<int32_t>(blockIdx.x * blockDim.x + threadIdx.x);
  if (c >= batch) return;
  active[c] = 1;
  steps_used[c] = 0;
  stopped[c] = 0;
  temperature[c] = t0;
}

// Seed of canvas k of each stream ("DiffusionGemma Lab", Figure 1: canvases
// chain block-autoregressively; each needs noise of its own).
__global__ void canvas_seeds_kernel(const uint64_t* __restrict__ seeds, int32_t batch, int32_t k,
                                    uint64_t* __restrict__ out) {
  const int32_t c = static_cast<int32_t>(blockIdx.x * blockDim.x + threadIdx.x);
  if (c >= batch) return;
  const uint64_t seed = seeds[c];
  if (k == 0) {
    out[c] = seed;
    return;
  }
  const Words4 w = philox4x32_10(static_cast<uint32_t>(k), 0u, 0u, kTagCanvas, static_cast<uint32_t>(seed),
                                 static_cast<uint32_t>(seed >> 32));
  out[c] = static_cast<uint64_t>(w.w[0]) | (static_cast<uint64_t>(w.w[1]) << 32);
}

__global__ void place_canvas_kernel(const int32_t* __restrict__ canvas, int32_t canvas_len, int64_t total,
                                    int32_t* __restrict__ tokens, int64_t ld, int64_t offset) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= total) return;
  const int64_t c = i / canvas_len;
  tokens[c * ld + offset + (i - c * canvas_len)] = canvas[i];
}

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int32_t n, uint32_t value) {
  const int32_t i = static_cast<int32_t>(blockIdx.x * blockDim.x + threadIdx.x);
  if (i < n) p[i] = value;
}

}  // namespace

hipError_t launch_fill_u32(uint32_t* p, int32_t n, uint32_t value, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int threads = 256;
  hipLaunchKernelGGL(fill_u32_kernel, dim3((n + threads - 1) / threads), dim3(threads), 0, stream, p, n, value);
  return hipGetLastError();
}

hipError_t launch_canvas_seeds(const uint64_t* seeds, int32_t batch, int32_t k, uint64_t* out,
                               hipStream_t stream) {
  const int threads = 256;
  hipLaunchKernelGGL(canvas_seeds_kernel, dim3((batch + threads - 1) / threads), dim3(threads), 0, stream,
                     seeds, batch, k, out);
  return hipGetLastError();
}

hipError_t launch_place_canvas(const int32_t* canvas, int32_t batch, int32_t canvas_len, int32_t* tokens,
                               int64_t ld, int64_t offset, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(batch) * canvas_len;
  const int threads = 256;
  hipLaunchKernelGGL(place_canvas_kernel, dim3(static_cast<unsigned>((total + threads - 1) / threads)),
                     dim3(threads), 0, stream, canvas, canvas_len, total, tokens, ld, offset);
  return hipGetLastError();
}

hipError_t launch_run_state_init(int32_t batch, uint8_t* active, int32_t* steps_used,
                                 uint8_t* stopped, float* temperature, float t0, hipStream_t stream) {
  const int threads = 256;
  hipLaunchKernelGGL(run_state_init_kernel, dim3((batch + threads - 1) / threads), dim3(threads), 0,
                     stream, batch, active, steps_used, stopped, temperature, t0);
  return hipGetLastError();
}

hipError_t launch_accept_renoise(const AcceptArgs& a, int32_t batch, hipStream_t stream) {
  hipLaunchKernelGGL(accept_renoise_kernel, dim3(batch), dim3(kAcceptThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_canvas_init(const uint64_t* seeds, int32_t batch, int32_t canvas_len,
                              int32_t vocab, int32_t* canvas, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(batch) * canvas_len;
  const int threads = 256;
  const unsigned blocks = static_cast<unsigned>((total + threads - 1) / threads);
  hipLaunchKernelGGL(canvas_init_kernel, dim3(blocks), dim3(threads), 0, stream, seeds,
                     canvas_len, vocab, total, canvas);
  return hipGetLastError();
}

}  // namespace dg
