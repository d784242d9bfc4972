// C ABI of the canvas sampler (include/dg_canvas.h): context and scratch,
// argument validation, kernel launches and the host-driven denoising loop.
#include "../../include/dg_canvas.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

struct dg_ctx {
  int device = 0;
  int32_t max_batch = 0;
  dg_params p{};
  int32_t nsplit_override = 0;
  int32_t nsplit_max = 8;
  int32_t cu_count = 0;                 // compute units of the device
  // device scratch
  dg::RowPartial* partials = nullptr;   // [max_rows * nsplit_max]
  float* entropy = nullptr;             // [max_rows]
  int32_t* argmax[2] = {nullptr, nullptr};
  int32_t* sample = nullptr;
  int32_t* canvas = nullptr;
  int32_t* finished = nullptr;          // [max_rows]: the last finished canvases of dg_generate
  float* sc_partials = nullptr;         // self-conditioning partial tiles
  int64_t sc_partial_floats = 0;
  uint64_t* seeds = nullptr;            // [max_batch]
  float* temperature = nullptr;
  uint8_t* active = nullptr;
  uint8_t* stop = nullptr;
  // pinned host staging
  uint8_t* stop_host = nullptr;
  uint8_t* active_host = nullptr;
  float* temp_host = nullptr;
  std::string err;
};

namespace {

// Rows are read through 32-bit buffer offsets; prefetches past a wave's last
// batch use offsets beyond this size.
constexpr int64_t kMaxRowBytes = 0x7FFF0000LL - 0x10000LL;

thread_local std::string g_err;

dg_status set_err(dg_ctx* ctx, dg_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  if (ctx)
    ctx->err = buf;
  else
    g_err = buf;
  return st;
}

#define DG_CHECK_HIP(ctx, call)                                                              \
  do {                                                                                       \
    hipError_t e_ = (call);                                                                  \
    if (e_ != hipSuccess)                                                                    \
      return set_err((ctx), DG_ERR_DEVICE, "%s failed: %s", #call, hipGetErrorString(e_));   \
  } while (0)

// Makes the context's device current for the duration of a call.
struct DeviceGuard {
  int prev = -1;
  bool ok = true;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) != hipSuccess) prev = -1;
    if (prev != dev) ok = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    int cur = -1;
    if (prev >= 0 && hipGetDevice(&cur) == hipSuccess && cur != prev) (void)hipSetDevice(prev);
  }
};

bool finite_positive(float x) { return std::isfinite(x) && x > 0.0f; }

dg_status check_params(dg_ctx* ctx, const dg_params* p) {
  if (!p) return set_err(ctx, DG_ERR_INVALID_ARG, "params is NULL");
  if (p->canvas_len < 1 || p->canvas_len > 256)
    return set_err(ctx, DG_ERR_INVALID_ARG, "params.canvas_len = %d is outside 1..256", p->canvas_len);
  if (p->vocab < 2)
    return set_err(ctx, DG_ERR_INVALID_ARG, "params.vocab = %d is below 2", p->vocab);
  if (!(p->entropy_bound >= 0.0f) || !std::isfinite(p->entropy_bound))
    return set_err(ctx, DG_ERR_INVALID_ARG,
                   "params.entropy_bound = %g must be finite and >= 0 (a negative bound could accept no position)",
                   static_cast<double>(p->entropy_bound));
  if (!finite_positive(p->temp_start))
    return set_err(ctx, DG_ERR_INVALID_ARG, "params.temp_start = %g must be finite and > 0",
                   static_cast<double>(p->temp_start));
  if (!finite_positive(p->temp_end))
    return set_err(ctx, DG_ERR_INVALID_ARG, "params.temp_end = %g must be finite and > 0",
                   static_cast<double>(p->temp_end));
  if (p->temp_steps < 1)
    return set_err(ctx, DG_ERR_INVALID_ARG, "params.temp_steps = %d must be >= 1", p->temp_steps);
  if (p->max_steps < 1)
    return set_err(ctx, DG_ERR_INVALID_ARG, "params.max_steps = %d must be >= 1", p->max_steps);
  if (!finite_positive(p->stop_mean_entropy))
    return set_err(ctx, DG_ERR_INVALID_ARG, "params.stop_mean_entropy = %g must be finite and > 0",
                   static_cast<double>(p->stop_mean_entropy));
  return DG_OK;
}

dg_status check_batch(dg_ctx* ctx, int32_t B) {
  if (B < 1 || B > ctx->max_batch)
    return set_err(ctx, DG_ERR_INVALID_ARG, "B = %d is outside 1..max_batch (%d)", B, ctx->max_batch);
  return DG_OK;
}

dg_status check_logits_v(dg_ctx* ctx, int32_t vocab, const void* logits, dg_dtype dtype, int64_t row_stride);

dg_status check_logits(dg_ctx* ctx, const void* logits, dg_dtype dtype, int64_t row_stride) {
  return check_logits_v(ctx, ctx->p.vocab, logits, dtype, row_stride);
}

dg_status check_logits_v(dg_ctx* ctx, int32_t vocab, const void* logits, dg_dtype dtype, int64_t row_stride) {
  if (!logits) return set_err(ctx, DG_ERR_INVALID_ARG, "logits is NULL");
  if (dtype != DG_DTYPE_F32 && dtype != DG_DTYPE_BF16)
    return set_err(ctx, DG_ERR_INVALID_ARG, "dtype = %d is not DG_DTYPE_F32 or DG_DTYPE_BF16",
                   static_cast<int>(dtype));
  if (row_stride < vocab)
    return set_err(ctx, DG_ERR_INVALID_ARG, "row_stride = %lld is below vocab (%d)",
                   static_cast<long long>(row_stride), vocab);
  if ((reinterpret_cast<uintptr_t>(logits) & 15u) != 0)
    return set_err(ctx, DG_ERR_UNSUPPORTED, "logits is not 16-byte aligned");
  const int64_t per16 = dtype == DG_DTYPE_BF16 ? 8 : 4;
  const int64_t row_bytes = static_cast<int64_t>(vocab) * (16 / per16);
  if (row_bytes > kMaxRowBytes)
    return set_err(ctx, DG_ERR_UNSUPPORTED,
                   "vocab = %d is too large for this dtype: a row must hold at most %lld bytes",
                   vocab, static_cast<long long>(kMaxRowBytes));
  if (row_stride % per16 != 0)
    return set_err(ctx, DG_ERR_UNSUPPORTED,
                   "row_stride = %lld must be a multiple of %lld elements (16 bytes)",
                   static_cast<long long>(row_stride), static_cast<long long>(per16));
  return DG_OK;
}

int32_t effective_nsplit(const dg_ctx* ctx, int32_t rows) {
  int32_t n = ctx->nsplit_override > 0 ? ctx->nsplit_override : dg::choose_nsplit(rows, ctx->p.vocab);
  if (n > ctx->nsplit_max) n = ctx->nsplit_max;
  return n < 1 ? 1 : n;
}

// Device resources a step's kernels work in: the context's scratch, or the
// static scratch of dg_sampler_step_noalloc.
struct StepScratch {
  int32_t nsplit;
  int32_t cu_count;
  dg::RowPartial* partials;
};

dg::StatsArgs make_stats_args(const dg_params& p, const StepScratch& sc, int32_t B, const void* logits,
                              int64_t row_stride, const float* temperature, int32_t step, const int32_t* steps,
                              const uint64_t* seeds, const uint8_t* active, float* entropy, int32_t* argmax,
                              int32_t* sample) {
  dg::StatsArgs a{};
  a.logits = logits;
  a.row_stride = row_stride;
  a.vocab = p.vocab;
  a.canvas_len = p.canvas_len;
  a.rows = B * p.canvas_len;
  a.nsplit = sc.nsplit;
  a.temperature = temperature;
  a.seeds = seeds;
  a.step = step;
  a.steps = steps;
  a.active = active;
  a.entropy = entropy;
  a.argmax = argmax;
  a.sample = sample;
  a.partials = sc.partials;
  a.row_grid = dg::stats_row_grid(a.rows, a.vocab, a.nsplit, active != nullptr, sc.cu_count);
  return a;
}

dg::StatsArgs stats_args(const dg_ctx* ctx, int32_t B, const void* logits, int64_t row_stride,
                         const float* temperature, int32_t step, const int32_t* steps,
                         const uint64_t* seeds, const uint8_t* active, float* entropy, int32_t* argmax,
                         int32_t* sample) {
  const StepScratch sc{effective_nsplit(ctx, B * ctx->p.canvas_len), ctx->cu_count, ctx->partials};
  return make_stats_args(ctx->p, sc, B, logits, row_stride, temperature, step, steps, seeds, active, entropy,
                         argmax, sample);
}

dg_status enqueue_stats(dg_ctx* ctx, int32_t B, const void* logits, dg_dtype dtype,
                        int64_t row_stride, const float* temperature, int32_t step,
                        const int32_t* steps, const uint64_t* seeds, const uint8_t* active,
                        float* entropy, int32_t* argmax, int32_t* sample, hipStream_t stream) {
  const dg::StatsArgs a = stats_args(ctx, B, logits, row_stride, temperature, step, steps, seeds, active,
                                     entropy, argmax, sample);
  DG_CHECK_HIP(ctx, dg::launch_canvas_stats(a, dtype == DG_DTYPE_BF16, stream));
  if (a.nsplit > 1) DG_CHECK_HIP(ctx, dg::launch_partials_merge(a, a.partials, a.nsplit, stream));
  return DG_OK;
}

dg::AcceptArgs make_accept_args(const dg_params& p, const float* entropy, const int32_t* argmax,
                                const int32_t* sample, int32_t step, const int32_t* steps,
                                const uint64_t* seeds, const int32_t* prev_argmax, const uint8_t* active,
                                const dg_step_out* out, bool copy_stats) {
  dg::AcceptArgs a{};
  a.entropy = entropy;
  a.argmax = argmax;
  a.sample = sample;
  a.seeds = seeds;
  a.prev_argmax = prev_argmax;
  a.active = active;
  a.step = step;
  a.steps = steps;
  a.canvas_len = p.canvas_len;
  a.vocab = p.vocab;
  a.bound = p.entropy_bound;
  a.stop_mean_entropy = p.stop_mean_entropy;
  a.canvas_out = out->canvas_out;
  if (copy_stats) {
    a.argmax_out = out->argmax_out;
    a.sample_out = out->sample_out;
    a.entropy_out = out->entropy_out;
  }
  a.accept_out = out->accept_out;
  a.n_accept_out = out->n_accept_out;
  a.mean_entropy_out = out->mean_entropy_out;
  a.stop_out = out->stop_out;
  return a;
}

dg::AcceptArgs accept_args(const dg_ctx* ctx, const float* entropy, const int32_t* argmax,
                           const int32_t* sample, int32_t step, const int32_t* steps,
                           const uint64_t* seeds, const int32_t* prev_argmax, const uint8_t* active,
                           const dg_step_out* out, bool copy_stats) {
  return make_accept_args(ctx->p, entropy, argmax, sample, step, steps, seeds, prev_argmax, active, out,
                          copy_stats);
}

dg_status enqueue_accept(dg_ctx* ctx, int32_t B, const float* entropy, const int32_t* argmax,
                         const int32_t* sample, int32_t step, const int32_t* steps,
                         const uint64_t* seeds, const int32_t* prev_argmax, const uint8_t* active,
                         const dg_step_out* out, bool copy_stats, hipStream_t stream) {
  const dg::AcceptArgs a = accept_args(ctx, entropy, argmax, sample, step, steps, seeds, prev_argmax,
                                       active, out, copy_stats);
  DG_CHECK_HIP(ctx, dg::launch_accept_renoise(a, B, stream));
  return DG_OK;
}

// One whole step: the statistics pass into (entropy, argmax, sample), then the
// per-canvas acceptance.
dg_status enqueue_step(dg_ctx* ctx, int32_t B, const void* logits, dg_dtype dtype, int64_t row_stride,
                       const float* temperature, int32_t step, const int32_t* steps,
                       const uint64_t* seeds, const int32_t* prev_argmax, const uint8_t* active,
                       float* entropy, int32_t* argmax, int32_t* sample, const dg_step_out* out,
                       bool copy_stats, hipStream_t stream) {
  const dg_status st = enqueue_stats(ctx, B, logits, dtype, row_stride, temperature, step, steps, seeds,
                                     active, entropy, argmax, sample, stream);
  if (st != DG_OK) return st;
  return enqueue_accept(ctx, B, entropy, argmax, sample, step, steps, seeds, prev_argmax, active, out,
                        copy_stats, stream);
}

// Operands of the LM-head product are read through 32-bit buffer offsets.
constexpr int64_t kMaxOperandBytes = 0x7FFF0000LL;

// The operands of the product (shared by both LM-head entry points).
dg_status check_lmhead_operands(dg_ctx* ctx, int32_t rows, const void* hidden, const void* weight,
                                int32_t hidden_dim) {
  if (!hidden) return set_err(ctx, DG_ERR_INVALID_ARG, "hidden is NULL");
  if (!weight) return set_err(ctx, DG_ERR_INVALID_ARG, "weight is NULL");
  if (hidden_dim < 1) return set_err(ctx, DG_ERR_INVALID_ARG, "hidden_dim = %d must be >= 1", hidden_dim);
  if (hidden_dim % 64 != 0)
    return set_err(ctx, DG_ERR_UNSUPPORTED, "hidden_dim = %d must be a multiple of 64", hidden_dim);
  if (ctx->p.vocab % 8 != 0)
    return set_err(ctx, DG_ERR_UNSUPPORTED, "vocab = %d must be a multiple of 8 for the LM head", ctx->p.vocab);
  if ((reinterpret_cast<uintptr_t>(hidden) & 15u) || (reinterpret_cast<uintptr_t>(weight) & 15u))
    return set_err(ctx, DG_ERR_UNSUPPORTED, "hidden and weight must be 16-byte aligned");
  if (static_cast<int64_t>(rows) * hidden_dim * 2 > kMaxOperandBytes)
    return set_err(ctx, DG_ERR_UNSUPPORTED, "hidden is too large: rows * hidden_dim * 2 = %lld bytes > %lld",
                   static_cast<long long>(static_cast<int64_t>(rows) * hidden_dim * 2),
                   static_cast<long long>(kMaxOperandBytes));
  if (static_cast<int64_t>(hidden_dim) * ctx->p.vocab * 2 > kMaxOperandBytes)
    return set_err(ctx, DG_ERR_UNSUPPORTED, "weight is too large: hidden_dim * vocab * 2 = %lld bytes > %lld",
                   static_cast<long long>(static_cast<int64_t>(hidden_dim) * ctx->p.vocab * 2),
                   static_cast<long long>(kMaxOperandBytes));
  return DG_OK;
}

dg_status check_lmhead(dg_ctx* ctx, int32_t rows, const void* hidden, const void* weight,
                       int32_t hidden_dim, const float* logits, int64_t ld_logits) {
  if (!hidden) return set_err(ctx, DG_ERR_INVALID_ARG, "hidden is NULL");
  if (!weight) return set_err(ctx, DG_ERR_INVALID_ARG, "weight is NULL");
  if (!logits) return set_err(ctx, DG_ERR_INVALID_ARG, "logits is NULL");
  if (hidden_dim < 1) return set_err(ctx, DG_ERR_INVALID_ARG, "hidden_dim = %d must be >= 1", hidden_dim);
  if (ld_logits < ctx->p.vocab)
    return set_err(ctx, DG_ERR_INVALID_ARG, "ld_logits = %lld is below vocab (%d)",
                   static_cast<long long>(ld_logits), ctx->p.vocab);
  const dg_status st = check_lmhead_operands(ctx, rows, hidden, weight, hidden_dim);
  if (st != DG_OK) return st;
  if (ld_logits % 4 != 0)
    return set_err(ctx, DG_ERR_UNSUPPORTED, "ld_logits = %lld must be a multiple of 4",
                   static_cast<long long>(ld_logits));
  if (reinterpret_cast<uintptr_t>(logits) & 15u)
    return set_err(ctx, DG_ERR_UNSUPPORTED, "logits must be 16-byte aligned");
  return DG_OK;
}

// Workspace of the fused LM-head step: one 40-byte partial per (row, tile),
// then one 32-bit running best score per row.
int64_t lmhead_partials_bytes(int32_t rows, int32_t vocab) {
  return static_cast<int64_t>(rows) * dg::lmhead_stats_tiles(vocab) * static_cast<int64_t>(sizeof(dg::RowPartial));
}

int64_t lmhead_workspace_bytes(int32_t rows, int32_t vocab) {
  return lmhead_partials_bytes(rows, vocab) + static_cast<int64_t>(rows) * 4;
}

dg_status enqueue_lmhead(dg_ctx* ctx, int32_t rows, const void* hidden, const void* weight,
                         int32_t hidden_dim, float* logits, int64_t ld_logits, hipStream_t stream) {
  dg::GemmArgs g{};
  g.hidden = hidden;
  g.weight = weight;
  g.logits = logits;
  g.ld_logits = ld_logits;
  g.rows = rows;
  g.hidden_dim = hidden_dim;
  g.vocab = ctx->p.vocab;
  DG_CHECK_HIP(ctx, dg::launch_lmhead_gemm(g, stream));
  return DG_OK;
}

template <typename T>
hipError_t dev_alloc(T** p, size_t n) {
  return hipMalloc(reinterpret_cast<void**>(p), n * sizeof(T) + 16);
}

void free_ctx(dg_ctx* c) {
  if (!c) return;
  hipFree(c->partials);
  hipFree(c->entropy);
  hipFree(c->argmax[0]);
  hipFree(c->argmax[1]);
  hipFree(c->sample);
  hipFree(c->canvas);
  hipFree(c->finished);
  hipFree(c->sc_partials);
  hipFree(c->seeds);
  hipFree(c->temperature);
  hipFree(c->active);
  hipFree(c->stop);
  hipHostFree(c->stop_host);
  hipHostFree(c->active_host);
  hipHostFree(c->temp_host);
  delete c;
}

}  // namespace

extern "C" {

const char* dg_version(void) { return "dgcanvas 0.1 (gfx950)"; }

dg_status dg_params_default(dg_params* p) {
  if (!p) return set_err(nullptr, DG_ERR_INVALID_ARG, "p is NULL");
  p->canvas_len = 256;
  p->vocab = 262144;
  p->entropy_bound = 0.1f;
  p->temp_start = 0.8f;
  p->temp_end = 0.4f;
  p->temp_steps = 48;
  p->max_steps = 48;
  p->stop_mean_entropy = 0.005f;
  return DG_OK;
}

dg_status dg_params_check(const dg_params* p) { return check_params(nullptr, p); }

const char* dg_last_error(const dg_ctx* ctx) { return ctx ? ctx->err.c_str() : g_err.c_str(); }

dg_status dg_get_params(const dg_ctx* ctx, dg_params* out) {
  if (!ctx) return set_err(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  if (!out) return set_err(const_cast<dg_ctx*>(ctx), DG_ERR_INVALID_ARG, "out is NULL");
  *out = ctx->p;
  return DG_OK;
}

dg_status dg_temperature(const dg_params* p, int32_t step, float* out) {
  dg_status st = check_params(nullptr, p);
  if (st != DG_OK) return st;
  if (step < 0) return set_err(nullptr, DG_ERR_INVALID_ARG, "step = %d is negative", step);
  if (!out) return set_err(nullptr, DG_ERR_INVALID_ARG, "out is NULL");
  const double t0 = p->temp_start, t1 = p->temp_end;
  if (p->temp_steps == 1) {
    *out = static_cast<float>(t0);
  } else {
    const int32_t s = step < p->temp_steps - 1 ? step : p->temp_steps - 1;
    *out = static_cast<float>(t0 + (t1 - t0) * static_cast<double>(s) / static_cast<double>(p->temp_steps - 1));
  }
  return DG_OK;
}

dg_status dg_create(dg_ctx** out, int device, int32_t max_batch, const dg_params* params) {
  if (!out) return set_err(nullptr, DG_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  dg_status st = check_params(nullptr, params);
  if (st != DG_OK) return st;
  if (max_batch < 1 || max_batch > 65536)
    return set_err(nullptr, DG_ERR_INVALID_ARG, "max_batch = %d is outside 1..65536", max_batch);
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev < 1)
    return set_err(nullptr, DG_ERR_DEVICE, "no HIP device is available");
  if (device < 0 || device >= ndev)
    return set_err(nullptr, DG_ERR_INVALID_ARG, "device = %d is outside 0..%d", device, ndev - 1);
  DeviceGuard guard(device);
  if (!guard.ok) return set_err(nullptr, DG_ERR_DEVICE, "hipSetDevice(%d) failed", device);

  dg_ctx* c = new dg_ctx();
  c->device = device;
  if (hipDeviceGetAttribute(&c->cu_count, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
    c->cu_count = 0;  // no row loop
  c->max_batch = max_batch;
  c->p = *params;
  const size_t rows = static_cast<size_t>(max_batch) * params->canvas_len;
  bool ok = dev_alloc(&c->partials, rows * c->nsplit_max) == hipSuccess &&
            dev_alloc(&c->entropy, rows) == hipSuccess &&
            dev_alloc(&c->argmax[0], rows) == hipSuccess && dev_alloc(&c->argmax[1], rows) == hipSuccess &&
            dev_alloc(&c->sample, rows) == hipSuccess && dev_alloc(&c->canvas, rows) == hipSuccess &&
            dev_alloc(&c->finished, rows) == hipSuccess && dev_alloc(&c->seeds, max_batch) == hipSuccess &&
            dev_alloc(&c->temperature, max_batch) == hipSuccess &&
            dev_alloc(&c->active, max_batch) == hipSuccess && dev_alloc(&c->stop, max_batch) == hipSuccess &&
            hipHostMalloc(reinterpret_cast<void**>(&c->stop_host), max_batch) == hipSuccess &&
            hipHostMalloc(reinterpret_cast<void**>(&c->active_host), max_batch) == hipSuccess &&
            hipHostMalloc(reinterpret_cast<void**>(&c->temp_host), sizeof(float) * max_batch) == hipSuccess;
  // partial tiles of the self-conditioning matmul: the most any batch up to
  // max_batch needs (none once the row tiles alone fill the target grid)
  for (int32_t b = 1; ok && b <= max_batch; ++b) {
    int32_t nslice = 0, kslice = 0;
    const int32_t rows_b = b * params->canvas_len;
    dg::choose_self_cond_slices(rows_b, params->vocab, &nslice, &kslice);
    if (nslice > 1) {
      const int64_t rows_pad = (rows_b + dg::kScRowTile - 1) / dg::kScRowTile * dg::kScRowTile;
      const int64_t need = static_cast<int64_t>(nslice) * rows_pad * 32;
      if (need > c->sc_partial_floats) c->sc_partial_floats = need;
    }
    if (nslice == 1) break;  // larger batches need no partials either
  }
  if (ok && c->sc_partial_floats > 0) ok = dev_alloc(&c->sc_partials, static_cast<size_t>(c->sc_partial_floats)) == hipSuccess;
  if (!ok) {
    free_ctx(c);
    (void)hipGetLastError();
    return set_err(nullptr, DG_ERR_OUT_OF_MEMORY, "could not allocate scratch for max_batch = %d", max_batch);
  }
  *out = c;
  return DG_OK;
}

dg_status dg_destroy(dg_ctx* ctx) {
  if (!ctx) return DG_OK;
  DeviceGuard guard(ctx->device);
  (void)hipDeviceSynchronize();
  free_ctx(ctx);
  return DG_OK;
}

dg_status dg_set_stats_split(dg_ctx* ctx, int32_t nsplit) {
  if (!ctx) return set_err(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  if (nsplit < 0 || nsplit > ctx->nsplit_max)
    return set_err(ctx, DG_ERR_INVALID_ARG, "nsplit = %d is outside 0..%d", nsplit, ctx->nsplit_max);
  ctx->nsplit_override = nsplit;
  return DG_OK;
}

dg_status dg_canvas_init(dg_ctx* ctx, int32_t B, const uint64_t* seeds, int32_t* canvas, void* stream) {
  if (!ctx) return set_err(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_batch(ctx, B);
  if (st != DG_OK) return st;
  if (!seeds) return set_err(ctx, DG_ERR_INVALID_ARG, "seeds is NULL");
  if (!canvas) return set_err(ctx, DG_ERR_INVALID_ARG, "canvas is NULL");
  DeviceGuard guard(ctx->device);
  DG_CHECK_HIP(ctx, dg::launch_canvas_init(seeds, B, ctx->p.canvas_len, ctx->p.vocab, canvas,
                                           static_cast<hipStream_t>(stream)));
  return DG_OK;
}

dg_status dg_canvas_stats(dg_ctx* ctx, int32_t B, const void* logits, dg_dtype dtype,
                          int64_t row_stride, const float* temperature, int32_t step,
                          const uint64_t* seeds, const uint8_t* active, float* entropy,
                          int32_t* argmax, int32_t* sample, void* stream) {
  if (!ctx) return set_err(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_batch(ctx, B);
  if (st != DG_OK) return st;
  if ((st = check_logits(ctx, logits, dtype, row_stride)) != DG_OK) return st;
  if (!temperature) return set_err(ctx, DG_ERR_INVALID_ARG, "temperature is NULL");
  if (step < 0) return set_err(ctx, DG_ERR_INVALID_ARG, "step = %d is negative", step);
  if (!seeds) return set_err(ctx, DG_ERR_INVALID_ARG, "seeds is NULL");
  if (!entropy) return set_err(ctx, DG_ERR_INVALID_ARG, "entropy is NULL");
  if (!argmax) return set_err(ctx, DG_ERR_INVALID_ARG, "argmax is NULL");
  if (!sample) return set_err(ctx, DG_ERR_INVALID_ARG, "sample is NULL");
  DeviceGuard guard(ctx->device);
  return enqueue_stats(ctx, B, logits, dtype, row_stride, temperature, step, nullptr, seeds, active,
                       entropy, argmax, sample, static_cast<hipStream_t>(stream));
}

dg_status dg_accept_renoise(dg_ctx* ctx, int32_t B, const float* entropy, const int32_t* argmax,
                            const int32_t* sample, int32_t step, const uint64_t* seeds,
                            const int32_t* prev_argmax, const uint8_t* active,
                            const dg_step_out* out, void* stream) {
  if (!ctx) return set_err(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_batch(ctx, B);
  if (st != DG_OK) return st;
  if (!entropy) return set_err(ctx, DG_ERR_INVALID_ARG, "entropy is NULL");
  if (!argmax) return set_err(ctx, DG_ERR_INVALID_ARG, "argmax is NULL");
  if (!sample) return set_err(ctx, DG_ERR_INVALID_ARG, "sample is NULL");
  if (step < 0) return set_err(ctx, DG_ERR_INVALID_ARG, "step = %d is negative", step);
  if (!seeds) return set_err(ctx, DG_ERR_INVALID_ARG, "seeds is NULL");
  if (!out) return set_err(ctx, DG_ERR_INVALID_ARG, "out is NULL");
  if (!out->canvas_out) return set_err(ctx, DG_ERR_INVALID_ARG, "out->canvas_out is NULL");
  DeviceGuard guard(ctx->device);
  return enqueue_accept(ctx, B, entropy, argmax, sample, step, nullptr, seeds, prev_argmax, active,
                        out, true, static_cast<hipStream_t>(stream));
}

dg_status dg_sampler_step(dg_ctx* ctx, int32_t B, const void* logits, dg_dtype dtype,
                          int64_t row_stride, const float* temperature, int32_t step,
                          const uint64_t* seeds, const int32_t* prev_argmax,
                          const uint8_t* active, const dg_step_out* out, void* stream) {
  if (!ctx) return set_err(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_batch(ctx, B);
  if (st != DG_OK) return st;
  if ((st = check_logits(ctx, logits, dtype, row_stride)) != DG_OK) return st;
  if (!temperature) return set_err(ctx, DG_ERR_INVALID_ARG, "temperature is NULL");
  if (step < 0) return set_err(ctx, DG_ERR_INVALID_ARG, "step = %d is negative", step);
  if (!seeds) return set_err(ctx, DG_ERR_INVALID_ARG, "seeds is NULL");
  if (!out) return set_err(ctx, DG_ERR_INVALID_ARG, "out is NULL");
  if (!out->canvas_out) return set_err(ctx, DG_ERR_INVALID_ARG, "out->canvas_out is NULL");
  DeviceGuard guard(ctx->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // statistics go straight to the caller's buffers when requested
  float* ent = out->entropy_out ? out->entropy_out : ctx->entropy;
  int32_t* am = out->argmax_out ? out->argmax_out : ctx->argmax[0];
  int32_t* smp = out->sample_out ? out->sample_out : ctx->sample;
  return enqueue_step(ctx, B, logits, dtype, row_stride, temperature, step, nullptr, seeds, prev_argmax,
                      active, ent, am, smp, out, false, s);
}

dg_status dg_lmhead_logits(dg_ctx* ctx, int32_t rows, const void* hidden, const void* weight,
                           int32_t hidden_dim, float* logits, int64_t ld_logits, void* stream) {
  if (!ctx) return set_err(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  if (rows < 1) return set_err(ctx, DG_ERR_INVALID_ARG, "rows = %d must be >= 1", rows);
  dg_status st = check_lmhead(ctx, rows, hidden, weight, hidden_dim, logits, ld_logits);
  if (st != DG_OK) return st;
  DeviceGuard guard(ctx->device);
  return enqueue_lmhead(ctx, rows, hidden, weight, hidden_dim, logits, ld_logits,
                        static_cast<hipStream_t>(stream));
}

dg_status dg_lmhead_workspace_bytes(const dg_ctx* ctx, int32_t B, int64_t* bytes) {
  if (!ctx) return set_err(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_ctx* c = const_cast<dg_ctx*>(ctx);
  const dg_status st = check_batch(c, B);
  if (st != DG_OK) return st;
  if (!bytes) return set_err(c, DG_ERR_INVALID_ARG, "bytes is NULL");
  *bytes = lmhead_workspace_bytes(B * ctx->p.canvas_len, ctx->p.vocab);
  return DG_OK;
}

dg_status dg_lmhead_sampler_step(dg_ctx* ctx, int32_t B, const void* hidden, const void* weight,
                                 int32_t hidden_dim, void* workspace, int64_t workspace_bytes,
                                 const float* temperature, int32_t step, const int32_t* steps,
                                 const uint64_t* seeds, const int32_t* prev_argmax, const uint8_t* active,
                                 const dg_step_out* out, void* stream) {
  if (!ctx) return set_err(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_batch(ctx, B);
  if (st != DG_OK) return st;
  const int32_t rows = B * ctx->p.canvas_len;
  if ((st = check_lmhead_operands(ctx, rows, hidden, weight, hidden_dim)) != DG_OK) return st;
  if (!workspace) return set_err(ctx, DG_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 15u)
    return set_err(ctx, DG_ERR_UNSUPPORTED, "workspace must be 16-byte aligned");
  const int64_t need = lmhead_workspace_bytes(rows, ctx->p.vocab);
  if (workspace_bytes < need)
    return set_err(ctx, DG_ERR_INVALID_ARG, "workspace_bytes = %lld is below the %lld bytes B = %d needs",
                   static_cast<long long>(workspace_bytes), static_cast<long long>(need), B);
  if (!temperature) return set_err(ctx, DG_ERR_INVALID_ARG, "temperature is NULL");
  if (step < 0) return set_err(ctx, DG_ERR_INVALID_ARG, "step = %d is negative", step);
  if (!seeds) return set_err(ctx, DG_ERR_INVALID_ARG, "seeds is NULL");
  if (!out) return set_err(ctx, DG_ERR_INVALID_ARG, "out is NULL");
  if (!out->canvas_out) return set_err(ctx, DG_ERR_INVALID_ARG, "out->canvas_out is NULL");
  DeviceGuard guard(ctx->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* ent = out->entropy_out ? out->entropy_out : ctx->entropy;
  int32_t* am = out->argmax_out ? out->argmax_out : ctx->argmax[0];
  int32_t* smp = out->sample_out ? out->sample_out : ctx->sample;

  dg::GemmArgs g{};
  g.hidden = hidden;
  g.weight = weight;
  g.rows = rows;
  g.hidden_dim = hidden_dim;
  g.vocab = ctx->p.vocab;
  g.canvas_len = ctx->p.canvas_len;
  g.temperature = temperature;
  g.seeds = seeds;
  g.step = step;
  g.steps = steps;
  g.active = active;
  g.partials = static_cast<dg::RowPartial*>(workspace);
  g.hint = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + lmhead_partials_bytes(rows, ctx->p.vocab));
  g.ntiles = dg::lmhead_stats_tiles(ctx->p.vocab);
  DG_CHECK_HIP(ctx, dg::launch_lmhead_stats(g, s));
  dg::StatsArgs a = stats_args(ctx, B, nullptr, ctx->p.vocab, temperature, step, steps, seeds, active, ent, am,
                               smp);
  DG_CHECK_HIP(ctx, dg::launch_partials_merge(a, g.partials, g.ntiles, s));
  return enqueue_accept(ctx, B, ent, am, smp, step, steps, seeds, prev_argmax, active, out, false, s);
}

}  // extern "C"

namespace {

// Arguments shared by the two run loops, checked before anything is enqueued.
dg_status check_run(dg_ctx* ctx, int32_t B, const uint64_t* seeds, bool has_denoise,
                    dg_dtype dtype, void* logits_scratch, int32_t* final_argmax,
                    int32_t* steps_used, uint8_t* stopped, const char* entry,
                    const char* final_name = "final_argmax") {
  if (!ctx) return set_err(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_batch(ctx, B);
  if (st != DG_OK) return st;
  if (!seeds) return set_err(ctx, DG_ERR_INVALID_ARG, "seeds is NULL");
  if (!has_denoise) return set_err(ctx, DG_ERR_INVALID_ARG, "denoise is NULL");
  const int64_t V = ctx->p.vocab;
  if ((st = check_logits(ctx, logits_scratch, dtype, V)) != DG_OK) {
    if (st == DG_ERR_UNSUPPORTED && std::strstr(ctx->err.c_str(), "row_stride"))
      return set_err(ctx, DG_ERR_UNSUPPORTED,
                     "vocab = %lld must be a multiple of %d for %s with this dtype",
                     static_cast<long long>(V), dtype == DG_DTYPE_BF16 ? 8 : 4, entry);
    if (std::strstr(ctx->err.c_str(), "logits"))
      return set_err(ctx, st, "logits_scratch: %s", ctx->err.c_str());
    return st;
  }
  if (!final_argmax) return set_err(ctx, DG_ERR_INVALID_ARG, "%s is NULL", final_name);
  if (!steps_used) return set_err(ctx, DG_ERR_INVALID_ARG, "steps_used is NULL");
  if (!stopped) return set_err(ctx, DG_ERR_INVALID_ARG, "stopped is NULL");
  return DG_OK;
}

dg_status check_selfcond(dg_ctx* ctx, const float* embed, int32_t d, const float* out, dg_dtype dtype,
                         int64_t row_stride) {
  // a wave reads 32 logits rows through one buffer resource: their bytes must
  // stay below 4 GiB
  const int64_t elem = dtype == DG_DTYPE_BF16 ? 2 : 4;
  if (row_stride * elem >= (int64_t{1} << 27))
    return set_err(ctx, DG_ERR_UNSUPPORTED, "self-conditioning needs row_stride * element size below 2^27 bytes "
                   "(got %lld elements)", static_cast<long long>(row_stride));
  if (!embed) return set_err(ctx, DG_ERR_INVALID_ARG, "embed is NULL");
  if (!out) return set_err(ctx, DG_ERR_INVALID_ARG, "selfcond output is NULL");
  if (d < 1 || d > 31) return set_err(ctx, DG_ERR_INVALID_ARG, "d = %d is outside 1..31", d);
  if ((reinterpret_cast<uintptr_t>(embed) & 3u) || (reinterpret_cast<uintptr_t>(out) & 3u))
    return set_err(ctx, DG_ERR_UNSUPPORTED, "embed and the selfcond output must be 4-byte aligned");
  return DG_OK;
}

dg_status enqueue_selfcond(dg_ctx* ctx, int32_t B, const void* logits, dg_dtype dtype, int64_t row_stride,
                           const float* temperature, const int32_t* argmax, const uint8_t* active,
                           const float* embed, int32_t d, float* out, hipStream_t s) {
  dg::SelfCondArgs a{};
  a.logits = logits;
  a.row_stride = row_stride;
  a.vocab = ctx->p.vocab;
  a.canvas_len = ctx->p.canvas_len;
  a.rows = B * ctx->p.canvas_len;
  a.temperature = temperature;
  a.argmax = argmax;
  a.active = active;
  a.embed = embed;
  a.d = d;
  a.out = out;
  dg::choose_self_cond_slices(a.rows, a.vocab, &a.nslice, &a.kslice);
  a.rows_pad = (a.rows + dg::kScRowTile - 1) / dg::kScRowTile * dg::kScRowTile;
  a.partials = ctx->sc_partials;
  if (a.nslice > 1 && static_cast<int64_t>(a.nslice) * a.rows_pad * 32 > ctx->sc_partial_floats)
    return set_err(ctx, DG_ERR_DEVICE, "self-conditioning scratch too small (internal error)");
  DG_CHECK_HIP(ctx, dg::launch_self_cond(a, dtype == DG_DTYPE_BF16, s));
  return DG_OK;
}

// The device-resident loop over the steps of B canvases: state initialised on
// the device, then per step the denoiser (denoise(step)), the statistics pass
// and the acceptance kernel, which advances the loop state itself. With
// check_every > 0 it waits for the active flags every check_every steps and
// stops once none is set; otherwise it never waits.
template <class Denoise>
dg_status resident_run(dg_ctx* ctx, int32_t B, const uint64_t* seeds, Denoise& denoise, dg_dtype dtype,
                       void* logits, int32_t* final_argmax, int32_t* steps_used, uint8_t* stopped,
                       int32_t check_every, hipStream_t s) {
  const int32_t L = ctx->p.canvas_len;
  const int64_t V = ctx->p.vocab;
  float t = 0.0f;
  (void)dg_temperature(&ctx->p, 0, &t);
  DG_CHECK_HIP(ctx, dg::launch_run_state_init(B, ctx->active, steps_used, stopped, ctx->temperature, t, s));
  DG_CHECK_HIP(ctx, dg::launch_canvas_init(seeds, B, L, ctx->p.vocab, ctx->canvas, s));
  for (int32_t step = 0; step < ctx->p.max_steps; ++step) {
    if (denoise(step) != 0) return set_err(ctx, DG_ERR_CALLBACK, "denoise callback failed at step %d", step);
    float t_next = 0.0f;
    (void)dg_temperature(&ctx->p, step + 1, &t_next);
    int32_t* am_cur = ctx->argmax[step & 1];
    const int32_t* am_prev = step > 0 ? ctx->argmax[(step - 1) & 1] : nullptr;
    dg_step_out o{};
    o.canvas_out = ctx->canvas;
    o.argmax_out = final_argmax;
    dg_status st = enqueue_stats(ctx, B, logits, dtype, V, ctx->temperature, step, nullptr, seeds, ctx->active,
                                 ctx->entropy, am_cur, ctx->sample, s);
    if (st != DG_OK) return st;
    dg::AcceptArgs a = accept_args(ctx, ctx->entropy, am_cur, ctx->sample, step, nullptr, seeds, am_prev,
                                   ctx->active, &o, true);
    a.run_active = ctx->active;
    a.run_steps_used = steps_used;
    a.run_stopped = stopped;
    a.run_temperature = ctx->temperature;
    a.run_next_temperature = t_next;
    DG_CHECK_HIP(ctx, dg::launch_accept_renoise(a, B, s));
    if (check_every > 0 && (step + 1) % check_every == 0 && step + 1 < ctx->p.max_steps) {
      DG_CHECK_HIP(ctx, hipMemcpyAsync(ctx->active_host, ctx->active, B, hipMemcpyDeviceToHost, s));
      DG_CHECK_HIP(ctx, hipStreamSynchronize(s));
      bool any = false;
      for (int32_t c = 0; c < B && !any; ++c) any = ctx->active_host[c] != 0;
      if (!any) break;
    }
  }
  return DG_OK;
}

}  // namespace

extern "C" {

dg_status dg_run_canvas(dg_ctx* ctx, int32_t B, const uint64_t* seeds, dg_denoise_fn denoise,
                        void* user, dg_dtype dtype, void* logits_scratch, int32_t* final_argmax,
                        int32_t* steps_used, uint8_t* stopped, void* stream) {
  dg_status st = check_run(ctx, B, seeds, denoise != nullptr, dtype, logits_scratch, final_argmax,
                           steps_used, stopped, "dg_run_canvas");
  if (st != DG_OK) return st;
  const int64_t V = ctx->p.vocab;
  DeviceGuard guard(ctx->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t L = ctx->p.canvas_len;

  for (int32_t c = 0; c < B; ++c) {
    steps_used[c] = 0;
    stopped[c] = 0;
    ctx->active_host[c] = 1;
  }
  DG_CHECK_HIP(ctx, hipMemcpyAsync(ctx->seeds, seeds, sizeof(uint64_t) * B, hipMemcpyHostToDevice, s));
  DG_CHECK_HIP(ctx, hipMemcpyAsync(ctx->active, ctx->active_host, B, hipMemcpyHostToDevice, s));
  DG_CHECK_HIP(ctx, dg::launch_canvas_init(ctx->seeds, B, L, ctx->p.vocab, ctx->canvas, s));

  int32_t remaining = B;
  for (int32_t step = 0; step < ctx->p.max_steps && remaining > 0; ++step) {
    if (denoise(user, step, ctx->canvas, ctx->active, logits_scratch, stream) != 0)
      return set_err(ctx, DG_ERR_CALLBACK, "denoise callback failed at step %d", step);
    float t = 0.0f;
    (void)dg_temperature(&ctx->p, step, &t);
    for (int32_t c = 0; c < B; ++c) ctx->temp_host[c] = t;
    DG_CHECK_HIP(ctx, hipMemcpyAsync(ctx->temperature, ctx->temp_host, sizeof(float) * B,
                                     hipMemcpyHostToDevice, s));
    int32_t* am_cur = ctx->argmax[step & 1];
    const int32_t* am_prev = step > 0 ? ctx->argmax[(step - 1) & 1] : nullptr;
    dg_step_out o{};
    o.canvas_out = ctx->canvas;           // the denoiser has consumed the old canvas
    o.argmax_out = final_argmax;          // holds each canvas's latest argmax canvas
    o.stop_out = ctx->stop;
    st = enqueue_step(ctx, B, logits_scratch, dtype, V, ctx->temperature, step, nullptr, ctx->seeds,
                      am_prev, ctx->active, ctx->entropy, am_cur, ctx->sample, &o, true, s);
    if (st != DG_OK) return st;
    DG_CHECK_HIP(ctx, hipMemcpyAsync(ctx->stop_host, ctx->stop, B, hipMemcpyDeviceToHost, s));
    DG_CHECK_HIP(ctx, hipStreamSynchronize(s));
    bool changed = false;
    for (int32_t c = 0; c < B; ++c) {
      if (!ctx->active_host[c]) continue;
      steps_used[c] = step + 1;
      if (ctx->stop_host[c]) {
        stopped[c] = 1;
        ctx->active_host[c] = 0;
        --remaining;
        changed = true;
      }
    }
    if (changed && remaining > 0)
      DG_CHECK_HIP(ctx, hipMemcpyAsync(ctx->active, ctx->active_host, B, hipMemcpyHostToDevice, s));
  }
  return DG_OK;
}

dg_status dg_run_canvas_resident(dg_ctx* ctx, int32_t B, const uint64_t* seeds,
                                 dg_denoise_fn denoise, void* user, dg_dtype dtype,
                                 void* logits_scratch, int32_t* final_argmax, int32_t* steps_used,
                                 uint8_t* stopped, int32_t check_every, void* stream) {
  dg_status st = check_run(ctx, B, seeds, denoise != nullptr, dtype, logits_scratch, final_argmax,
                           steps_used, stopped, "dg_run_canvas_resident");
  if (st != DG_OK) return st;
  if (check_every < 0)
    return set_err(ctx, DG_ERR_INVALID_ARG, "check_every = %d must be >= 0", check_every);
  DeviceGuard guard(ctx->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto call = [&](int32_t step) {
    return denoise(user, step, ctx->canvas, ctx->active, logits_scratch, stream);
  };
  st = resident_run(ctx, B, seeds, call, dtype, logits_scratch, final_argmax, steps_used, stopped,
                    check_every, s);
  if (st == DG_OK && check_every > 0) DG_CHECK_HIP(ctx, hipStreamSynchronize(s));
  return st;
}

dg_status dg_generate(dg_ctx* ctx, int32_t B, const uint64_t* seeds, int32_t n_canvases,
                      dg_block_denoise_fn denoise, dg_cache_fn cache_update, void* user, dg_dtype dtype,
                      void* logits_scratch, int32_t* tokens, int32_t* steps_used, uint8_t* stopped,
                      int32_t check_every, void* stream) {
  dg_status st = check_run(ctx, B, seeds, denoise != nullptr, dtype, logits_scratch, tokens, steps_used,
                           stopped, "dg_generate", "tokens");
  if (st != DG_OK) return st;
  if (check_every < 0)
    return set_err(ctx, DG_ERR_INVALID_ARG, "check_every = %d must be >= 0", check_every);
  const int32_t L = ctx->p.canvas_len;
  if (n_canvases < 1 || static_cast<int64_t>(n_canvases) * L > INT32_MAX)
    return set_err(ctx, DG_ERR_INVALID_ARG, "n_canvases = %d must be in 1..%d", n_canvases, INT32_MAX / L);
  DeviceGuard guard(ctx->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t ld = static_cast<int64_t>(n_canvases) * L;
  for (int32_t k = 0; k < n_canvases; ++k) {
    DG_CHECK_HIP(ctx, dg::launch_canvas_seeds(seeds, B, k, ctx->seeds, s));
    auto call = [&](int32_t step) {
      return denoise(user, k, step, ctx->canvas, ctx->active, logits_scratch, stream);
    };
    st = resident_run(ctx, B, ctx->seeds, call, dtype, logits_scratch, ctx->finished,
                      steps_used + static_cast<int64_t>(k) * B, stopped + static_cast<int64_t>(k) * B,
                      check_every, s);
    if (st != DG_OK) return st;
    DG_CHECK_HIP(ctx, dg::launch_place_canvas(ctx->finished, B, L, tokens, ld, static_cast<int64_t>(k) * L, s));
    if (cache_update && cache_update(user, k, ctx->finished, stream) != 0)
      return set_err(ctx, DG_ERR_CALLBACK, "cache_update callback failed after canvas %d", k);
  }
  if (check_every > 0) DG_CHECK_HIP(ctx, hipStreamSynchronize(s));
  return DG_OK;
}

dg_status dg_self_condition(dg_ctx* ctx, int32_t B, const void* logits, dg_dtype dtype, int64_t row_stride,
                           const float* temperature, const int32_t* argmax, const float* embed, int32_t d,
                           float* out, void* stream) {
  if (!ctx) return set_err(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_batch(ctx, B);
  if (st != DG_OK) return st;
  if ((st = check_logits(ctx, logits, dtype, row_stride)) != DG_OK) return st;
  if (!temperature) return set_err(ctx, DG_ERR_INVALID_ARG, "temperature is NULL");
  if (!argmax) return set_err(ctx, DG_ERR_INVALID_ARG, "argmax is NULL");
  if ((st = check_selfcond(ctx, embed, d, out, dtype, row_stride)) != DG_OK) return st;
  DeviceGuard guard(ctx->device);
  return enqueue_selfcond(ctx, B, logits, dtype, row_stride, temperature, argmax, nullptr, embed, d, out,
                          static_cast<hipStream_t>(stream));
}

dg_status dg_sampler_step_selfcond(dg_ctx* ctx, int32_t B, const void* logits, dg_dtype dtype,
                                   int64_t row_stride, const float* temperature, int32_t step,
                                   const uint64_t* seeds, const int32_t* prev_argmax, const uint8_t* active,
                                   const float* embed, int32_t d, float* selfcond_out, const dg_step_out* out,
                                   void* stream) {
  if (!ctx) return set_err(nullptr, DG_ERR_INVALID_ARG, "ctx is NULL");
  dg_status st = check_batch(ctx, B);
  if (st != DG_OK) return st;
  if ((st = check_logits(ctx, logits, dtype, row_stride)) != DG_OK) return st;
  if (!temperature) return set_err(ctx, DG_ERR_INVALID_ARG, "temperature is NULL");
  if (step < 0) return set_err(ctx, DG_ERR_INVALID_ARG, "step = %d is negative", step);
  if (!seeds) return set_err(ctx, DG_ERR_INVALID_ARG, "seeds is NULL");
  if (!out) return set_err(ctx, DG_ERR_INVALID_ARG, "out is NULL");
  if (!out->canvas_out) return set_err(ctx, DG_ERR_INVALID_ARG, "out->canvas_out is NULL");
  if ((st = check_selfcond(ctx, embed, d, selfcond_out, dtype, row_stride)) != DG_OK) return st;
  DeviceGuard guard(ctx->device);
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* ent = out->entropy_out ? out->entropy_out : ctx->entropy;
  int32_t* am = out->argmax_out ? out->argmax_out : ctx->argmax[0];
  int32_t* smp = out->sample_out ? out->sample_out : ctx->sample;
  st = enqueue_stats(ctx, B, logits, dtype, row_stride, temperature, step, nullptr, seeds, active, ent, am,
                     smp, s);
  if (st != DG_OK) return st;
  st = enqueue_selfcond(ctx, B, logits, dtype, row_stride, temperature, am, active, embed, d, selfcond_out, s);
  if (st != DG_OK) return st;
  return enqueue_accept(ctx, B, ent, am, smp, step, nullptr, seeds, prev_argmax, active, out, false, s);
}

dg_status dg_tokens_per_forward(const int32_t* steps_used, int32_t n_canvases, int32_t B,
                                int32_t canvas_len, double* tpf, double* tpf_all) {
  if (!steps_used) return set_err(nullptr, DG_ERR_INVALID_ARG, "steps_used is NULL");
  if (n_canvases < 1) return set_err(nullptr, DG_ERR_INVALID_ARG, "n_canvases = %d must be >= 1", n_canvases);
  if (B < 1) return set_err(nullptr, DG_ERR_INVALID_ARG, "B = %d must be >= 1", B);
  if (canvas_len < 1) return set_err(nullptr, DG_ERR_INVALID_ARG, "canvas_len = %d must be >= 1", canvas_len);
  for (int64_t i = 0; i < static_cast<int64_t>(n_canvases) * B; ++i)
    if (steps_used[i] < 0)
      return set_err(nullptr, DG_ERR_INVALID_ARG, "steps_used[%lld] = %d is negative",
                     static_cast<long long>(i), steps_used[i]);
  int64_t all = 0;
  for (int32_t c = 0; c < B; ++c) {
    int64_t fwd = n_canvases;  // one cache-update forward per canvas
    for (int32_t k = 0; k < n_canvases; ++k) fwd += steps_used[static_cast<int64_t>(k) * B + c];
    all += fwd;
    if (tpf) tpf[c] = static_cast<double>(n_canvases) * canvas_len / static_cast<double>(fwd);
  }
  if (tpf_all) tpf_all[0] = static_cast<double>(n_canvases) * B * canvas_len / static_cast<double>(all);
  return DG_OK;
}

}  // extern "C"

// ---- One step that allocates nothing (dg_sampler_step_noalloc) ----
//
// The step's intermediate statistics and split-row partials live in
// `scratch`, a static array of device memory that every GPU the library runs
// on holds until the process ends. Host code never passes the array's name to
// a kernel: on the host that name is a stand-in, not a device address. Its
// address on each device is taken once, with the device current, through
// hipGetSymbolAddress and used from then on.

namespace {

constexpr int32_t kNoAllocMaxRows = 16384;     // B * L at most: 64 canvases of 256 positions
constexpr int32_t kNoAllocMaxPartials = 256;   // split rows: rows * nsplit <= 128 when nsplit > 1
constexpr size_t kNoAllocEntropyOff = 0;
constexpr size_t kNoAllocArgmaxOff = kNoAllocEntropyOff + sizeof(float) * kNoAllocMaxRows;
constexpr size_t kNoAllocSampleOff = kNoAllocArgmaxOff + sizeof(int32_t) * kNoAllocMaxRows;
constexpr size_t kNoAllocPartialOff = kNoAllocSampleOff + sizeof(int32_t) * kNoAllocMaxRows;
constexpr size_t kNoAllocBytes = kNoAllocPartialOff + sizeof(dg::RowPartial) * kNoAllocMaxPartials;
static_assert(kNoAllocPartialOff % 256 == 0, "partials stay 256-byte aligned");

}  // namespace

static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

namespace {

constexpr int kNoAllocMaxDevices = 64;

struct NoAllocDevice {
  unsigned char* base = nullptr;   // device address of `scratch` on this device
  int32_t cu_count = 0;
};

std::mutex g_noalloc_mu;
NoAllocDevice g_noalloc[kNoAllocMaxDevices];

// The current device's copy of `scratch`, looked up on the first call on each
// device (with that device current) and kept for the process.
dg_status noalloc_device(NoAllocDevice* out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return set_err(nullptr, DG_ERR_DEVICE, "no current HIP device");
  if (dev >= kNoAllocMaxDevices)
    return set_err(nullptr, DG_ERR_UNSUPPORTED, "device %d is beyond the %d devices supported", dev,
                   kNoAllocMaxDevices);
  std::lock_guard<std::mutex> lock(g_noalloc_mu);
  NoAllocDevice& d = g_noalloc[dev];
  if (d.base == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return set_err(nullptr, DG_ERR_DEVICE, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cu = 0;
    d.cu_count = cu;
    d.base = static_cast<unsigned char*>(p);
  }
  *out = d;
  return DG_OK;
}

}  // namespace

extern "C" {

dg_status dg_sampler_step_noalloc(const dg_params* params, int32_t B, const void* logits, dg_dtype dtype,
                                  int64_t row_stride, const float* temperature, int32_t step,
                                  const uint64_t* seeds, const int32_t* prev_argmax, const uint8_t* active,
                                  const dg_step_out* out, void* stream) {
  dg_status st = check_params(nullptr, params);
  if (st != DG_OK) return st;
  const dg_params& p = *params;
  if (B < 1) return set_err(nullptr, DG_ERR_INVALID_ARG, "B = %d must be >= 1", B);
  if (static_cast<int64_t>(B) * p.canvas_len > kNoAllocMaxRows)
    return set_err(nullptr, DG_ERR_INVALID_ARG,
                   "B * canvas_len = %lld exceeds the %d rows of the static scratch",
                   static_cast<long long>(B) * p.canvas_len, kNoAllocMaxRows);
  if ((st = check_logits_v(nullptr, p.vocab, logits, dtype, row_stride)) != DG_OK) return st;
  if (!temperature) return set_err(nullptr, DG_ERR_INVALID_ARG, "temperature is NULL");
  if (step < 0) return set_err(nullptr, DG_ERR_INVALID_ARG, "step = %d is negative", step);
  if (!seeds) return set_err(nullptr, DG_ERR_INVALID_ARG, "seeds is NULL");
  if (!out) return set_err(nullptr, DG_ERR_INVALID_ARG, "out is NULL");
  if (!out->canvas_out) return set_err(nullptr, DG_ERR_INVALID_ARG, "out->canvas_out is NULL");
  NoAllocDevice d;
  if ((st = noalloc_device(&d)) != DG_OK) return st;
  const int32_t rows = B * p.canvas_len;
  int32_t nsplit = dg::choose_nsplit(rows, p.vocab);
  if (nsplit > 1 && static_cast<int64_t>(rows) * nsplit > kNoAllocMaxPartials)
    return set_err(nullptr, DG_ERR_DEVICE, "split of %d rows over %d workgroups exceeds the static scratch "
                   "(internal error)", rows, nsplit);
  StepScratch sc{nsplit, d.cu_count, reinterpret_cast<dg::RowPartial*>(d.base + kNoAllocPartialOff)};
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* ent = out->entropy_out ? out->entropy_out : reinterpret_cast<float*>(d.base + kNoAllocEntropyOff);
  int32_t* am = out->argmax_out ? out->argmax_out : reinterpret_cast<int32_t*>(d.base + kNoAllocArgmaxOff);
  int32_t* smp = out->sample_out ? out->sample_out : reinterpret_cast<int32_t*>(d.base + kNoAllocSampleOff);
  const dg::StatsArgs a = make_stats_args(p, sc, B, logits, row_stride, temperature, step, nullptr, seeds, active,
                                          ent, am, smp);
  DG_CHECK_HIP(nullptr, dg::launch_canvas_stats(a, dtype == DG_DTYPE_BF16, s));
  if (a.nsplit > 1) DG_CHECK_HIP(nullptr, dg::launch_partials_merge(a, a.partials, a.nsplit, s));
  const dg::AcceptArgs acc = make_accept_args(p, ent, am, smp, step, nullptr, seeds, prev_argmax, active, out, false);
  DG_CHECK_HIP(nullptr, dg::launch_accept_renoise(acc, B, s));
  return DG_OK;
}

}  // extern "C"
