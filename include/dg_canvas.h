/*
 * dg_canvas.h — C ABI of the MI355X (gfx950) per-step canvas sampler used by
 * block-diffusion decoding.
 *
 * One sampler step turns the denoiser's logits for B canvases of L positions
 * ([B*L, V] rows, V contiguous) into the next canvas and a stop decision:
 *
 *   per position  temperature-scaled softmax, its entropy (nats), the argmax of
 *                 the raw logits and one multinomial sample;
 *   per canvas    sort the L entropies ascending, accept the longest sorted
 *                 prefix whose cumulative entropy minus its largest entropy is
 *                 at most b, write the sample at accepted positions and a fresh
 *                 uniform vocabulary token everywhere else, and evaluate the
 *                 adaptive stop (argmax canvas unchanged from the previous step
 *                 and mean entropy below a threshold).
 *
 * Sources (web pages on DiffusionGemma):
 *   "DiffusionGemma Lab" (shadowgraph.io), §2 "The generation algorithm, as
 *       written in the code", items 1-5 and 7; §3 EXP A and EXP B; "Side
 *       finding: an upstream bug".
 *   "DiffusionGemma: Parallel Denoising From an Autoregressive Checkpoint"
 *       (boxwrench.dev), "Finding": Algorithm 1 (entropy-bounded acceptance,
 *       temperature annealing, adaptive stopping), the architecture paragraph
 *       (canvases appended to the encoder's cache; the self-conditioning
 *       block) and the hardware paragraph (the sampling stage; tokens per
 *       forward pass).
 *   "DiffusionGemma: When the LLM Stops Writing Left to Right" (LunarOps),
 *       "What DiffusionGemma Actually Is": block-autoregressive multi-canvas
 *       sampling.
 *
 * The pages fix the rules but not how the multinomial sample or the noise is
 * drawn. This library fixes one random protocol so that its integer outputs
 * are reproducible bit for bit (a "two-level Gumbel-max" over vocabulary
 * blocks driven by Philox4x32-10, Salmon et al., SC'11):
 *
 *   key      = (low 32 bits of seed_c, high 32 bits of seed_c) for canvas c
 *   counter  = (c0, position l, step s, tag)
 *   tags     INIT = 0, BLOCK = 1, ELEM = 2, RENOISE = 3, CANVAS = 4
 *   uniform  U(w) = (2*(w >> 9) + 1) * 2^-24   (in (0,1), exact in fp32)
 *   Gumbel   G(w) = -ln(-ln U(w))
 *   blocks   vocabulary id v lies in block j = 64*(v >> 12) + ((v >> 3) & 63):
 *            a block is one 8-id slot of each of the 8 consecutive 512-id
 *            stripes of a 4096-id chunk (64 ids when full).
 *   sample   j* = argmax_j (LSE_{v in j}(z_v/T) + G_j), G_j = G(word (j>>9)&3
 *            of (j & ~0x600, l, s, BLOCK)): one call serves the four blocks
 *            whose numbers differ only in bits 9-10;
 *            y  = argmax_{v in j*} (z_v/T + G(word v&3 of (v>>2, l, s, ELEM)));
 *            ties go to the lowest j, then the lowest v. By the Gumbel-max
 *            property P(y = v) = softmax(z/T)_v exactly.
 *   uniform token for position l at step s: floor(w0 * V / 2^32) with
 *            w0 from (0, l, s, RENOISE); initial canvas: (0, l, 0, INIT).
 *   temperature at step s: (float)(T0 + (T1-T0) * min(s, S-1) / (S-1)),
 *            evaluated in double, T0 when S == 1.
 *   seed of canvas k >= 1 of a block-autoregressive stream (dg_generate):
 *            words 0 (low) and 1 (high) of (k, 0, 0, CANVAS = 4) under the
 *            stream's key; canvas 0 uses the stream's seed.
 *
 * Conventions for every entry point
 *   - Device pointers are addresses in the memory of the context's device;
 *     host pointers are ordinary CPU memory. Each argument says which.
 *   - The caller owns every buffer it passes. The context owns only its scratch,
 *     sized at dg_create from max_batch and params.vocab; no call allocates
 *     device memory after dg_create.
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls enqueue work on
 *     it and return without waiting, except dg_run_canvas, which waits once per
 *     step for the stop flags, and dg_run_canvas_resident with check_every > 0,
 *     which waits once per check_every steps.
 *   - Every argument is validated before anything is enqueued. On any error
 *     nothing is written to any output; dg_last_error() names the offending
 *     argument or the failing runtime call.
 *   - A context is used by one host thread and one stream at a time.
 *   - Logits must be finite or -inf (probability 0). A row needs at least one
 *     finite logit. NaN and +inf are outside the contract.
 */
#ifndef DG_CANVAS_H
#define DG_CANVAS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct dg_ctx dg_ctx;

typedef enum {
  DG_OK = 0,
  DG_ERR_INVALID_ARG = 1,   /* an argument is out of range or NULL       */
  DG_ERR_UNSUPPORTED = 2,   /* valid request outside what is implemented */
  DG_ERR_OUT_OF_MEMORY = 3, /* dg_create could not allocate its scratch  */
  DG_ERR_DEVICE = 4,        /* a HIP runtime call failed                 */
  DG_ERR_CALLBACK = 5       /* the denoiser callback returned non-zero   */
} dg_status;

typedef enum { DG_DTYPE_F32 = 0, DG_DTYPE_BF16 = 1 } dg_dtype;

/* Sampler parameters. Defaults are the official ones reported on the pages:
 * canvas of 256 ("DiffusionGemma Lab", §1), bound b = 0.1 (§2 item 2),
 * temperature 0.8 -> 0.4 (§2 item 4), stop at mean entropy < 0.005 (§2 item 3),
 * cap of 48 steps (boxwrench.dev, Algorithm 1, adaptive stopping). */
typedef struct {
  int32_t canvas_len;       /* L, 1..256                                   */
  int32_t vocab;            /* V, 2..2^31-1                                */
  float entropy_bound;      /* b >= 0 (b < 0 could accept nothing)         */
  float temp_start;         /* T0 > 0                                      */
  float temp_end;           /* T1 > 0                                      */
  int32_t temp_steps;       /* S >= 1: steps over which T goes T0 -> T1    */
  int32_t max_steps;        /* step cap >= 1                               */
  float stop_mean_entropy;  /* > 0; stop needs mean entropy strictly below */
} dg_params;

/* Fills *p with the defaults above (vocab = 262144, temp_steps = max_steps =
 * 48). Returns DG_ERR_INVALID_ARG if p is NULL. */
dg_status dg_params_default(dg_params* p);

/* Checks every field of *p against the ranges above. The error message names
 * the first offending field (the pages report an upstream validator whose
 * error path named the wrong attribute: "DiffusionGemma Lab", "Side finding").
 * Host only; no context needed. Message via dg_last_error(NULL). */
dg_status dg_params_check(const dg_params* p);

/* Creates a context on HIP device `device` for batches of up to max_batch
 * canvases (1..65536) with parameters *params (copied). Allocates the device
 * scratch (per-row partials, argmax ping-pong buffers) and a small
 * pinned host buffer. On failure *out is set to NULL and the message is
 * available from dg_last_error(NULL). */
dg_status dg_create(dg_ctx** out, int device, int32_t max_batch, const dg_params* params);

/* Frees the context and its scratch. NULL is accepted. Waits for the device. */
dg_status dg_destroy(dg_ctx* ctx);

/* Message of the last failed call on ctx, or of the last failed context-free
 * call (dg_create, dg_params_check, dg_temperature) of this thread when ctx is
 * NULL. Never NULL; "" when there was no error. Valid until the next call. */
const char* dg_last_error(const dg_ctx* ctx);

/* Copy of the context's parameters. */
dg_status dg_get_params(const dg_ctx* ctx, dg_params* out);

/* Temperature at step `step` (>= 0) of the linear schedule of *p
 * ("DiffusionGemma Lab", §2 item 4; boxwrench.dev, Algorithm 1, temperature
 * annealing): (float)(T0 + (T1-T0)*min(step,S-1)/(S-1)) in double; T0 if S==1.
 * Host only. */
dg_status dg_temperature(const dg_params* p, int32_t step, float* out);

/* Sets how many workgroups share one row in the statistics pass (1..8), or 0
 * for the automatic choice (the default). Meant for tuning and tests: the
 * argmax does not depend on it, and the other outputs only through
 * last-bit rounding of the block scores and entropies. */
dg_status dg_set_stats_split(dg_ctx* ctx, int32_t nsplit);

/* Initial canvas ("DiffusionGemma Lab", §2 item 1: uniform random vocabulary
 * tokens, not [MASK]). canvas[c*L + l] = floor(w0 * V / 2^32), w0 = word 0 of
 * Philox(seed_c; (0, l, 0, INIT)).
 *   B       1..max_batch
 *   seeds   device, uint64 [B]
 *   canvas  device, int32 [B, L], written */
dg_status dg_canvas_init(dg_ctx* ctx, int32_t B, const uint64_t* seeds, int32_t* canvas,
                         void* stream);

/* Per-position statistics only (the streaming pass of a step). For every row
 * r = c*L + l of an active canvas c:
 *   entropy[r] = H of softmax(z_r / T_c), nats, >= +0  (fp32)
 *   argmax[r]  = lowest v with z_rv = max_v z_rv (raw logits)
 *   sample[r]  = the protocol's two-level Gumbel-max draw at step `step`
 * Rows of inactive canvases are not written. Arguments:
 *   logits       device, [B*L rows, row_stride elements] of `dtype`; base
 *                16-byte aligned; row_stride >= V and a multiple of 8 (bf16)
 *                or 4 (fp32), and V * element size below 2^31 - 2^17 bytes,
 *                else DG_ERR_UNSUPPORTED
 *   temperature  device, fp32 [B], each > 0 and finite
 *   step         >= 0 (enters the random counters)
 *   seeds        device, uint64 [B]
 *   active       device, uint8 [B] (0 = skip canvas) or NULL = all active.
 *                The kernels read each flag through the aligned 32-bit word
 *                that holds it (a scalar load), so they may read up to 3
 *                bytes before the array's start and 3 after its end, all
 *                inside the same 4-byte-aligned words; the array must lie in
 *                readable device memory that those words cover (any device
 *                allocation does), and the extra bytes are never used
 *   entropy, argmax, sample  device outputs [B*L]; none may be NULL */
dg_status dg_canvas_stats(dg_ctx* ctx, int32_t B, const void* logits, dg_dtype dtype,
                          int64_t row_stride, const float* temperature, int32_t step,
                          const uint64_t* seeds, const uint8_t* active, float* entropy,
                          int32_t* argmax, int32_t* sample, void* stream);

/* Outputs of a step. Device pointers, caller-owned. canvas_out is required;
 * any other may be NULL (not requested). Shapes: [B, L] or [B]. */
typedef struct {
  int32_t* canvas_out;       /* next canvas: sample at accepted positions, else a uniform token */
  int32_t* argmax_out;       /* argmax canvas of this step (the decoded output when stopping)  */
  int32_t* sample_out;       /* multinomial sample per position                                 */
  uint8_t* accept_out;       /* 1 at accepted positions                                         */
  float* entropy_out;        /* per-position entropy, nats                                      */
  int32_t* n_accept_out;     /* [B] number of accepted positions (>= 1)                         */
  float* mean_entropy_out;   /* [B] mean of the L entropies                                     */
  uint8_t* stop_out;         /* [B] adaptive stop fired at this step                            */
} dg_step_out;

/* Acceptance, renoise and stop only, from given per-position statistics
 * (entropy, argmax, sample: device [B*L]). Follows "DiffusionGemma Lab", §2
 * items 2, 3, 5 and boxwrench.dev Algorithm 1:
 *   order positions by (entropy, position) ascending; with C_i the inclusive
 *   cumulative sum and M_i the running maximum over that order, accept the
 *   longest prefix with C_i - M_i <= b (always >= 1 position);
 *   canvas_out = sample where accepted, else floor(w0*V/2^32) with w0 from
 *   Philox(seed_c; (0, l, step, RENOISE));
 *   stop = (prev_argmax given) && argmax == prev_argmax at all L positions
 *          && mean entropy < stop_mean_entropy.
 *   prev_argmax  device int32 [B, L], or NULL when there is no previous step
 *   active       device uint8 [B] or NULL = all active; inactive canvases are
 *                left untouched in every output. */
dg_status dg_accept_renoise(dg_ctx* ctx, int32_t B, const float* entropy, const int32_t* argmax,
                            const int32_t* sample, int32_t step, const uint64_t* seeds,
                            const int32_t* prev_argmax, const uint8_t* active,
                            const dg_step_out* out, void* stream);

/* One full sampler step: dg_canvas_stats followed by dg_accept_renoise, with
 * the statistics kept in the context's scratch unless out requests them.
 * Arguments as for those two calls. */
dg_status dg_sampler_step(dg_ctx* ctx, int32_t B, const void* logits, dg_dtype dtype,
                          int64_t row_stride, const float* temperature, int32_t step,
                          const uint64_t* seeds, const int32_t* prev_argmax,
                          const uint8_t* active, const dg_step_out* out, void* stream);

/* Denoiser callback of dg_run_canvas: must enqueue on `stream` the writing of
 * logits for step `step` into logits_dev ([B*L, V] rows of the run's dtype,
 * row stride V) from the current canvas (device int32 [B, L]); canvases with
 * active_dev[c] == 0 may be skipped. Returns 0 on success. */
typedef int (*dg_denoise_fn)(void* user, int32_t step, const int32_t* canvas_dev,
                             const uint8_t* active_dev, void* logits_dev, void* stream);

/* Whole denoising of B canvases ("DiffusionGemma Lab", §2 items 1-5;
 * boxwrench.dev Algorithm 1): initial uniform canvas, then for
 * s = 0 .. max_steps-1: callback, T_s from the schedule, one step over the
 * active canvases; a canvas whose stop fires is finished with that step's
 * argmax canvas and leaves the batch; after max_steps the remaining canvases
 * are finished with the last argmax canvas.
 *   seeds           host uint64 [B]
 *   logits_scratch  device, [B*L, V] of dtype (16-byte aligned; V a multiple of
 *                   8 for bf16 or 4 for fp32), written by the callback
 *   final_argmax    device int32 [B, L], written
 *   steps_used      host int32 [B], written (1..max_steps)
 *   stopped         host uint8 [B], written: 1 if the adaptive stop fired
 * Returns DG_ERR_CALLBACK if the callback fails; steps_used then holds the
 * steps completed so far (finished canvases keep their values). */
dg_status dg_run_canvas(dg_ctx* ctx, int32_t B, const uint64_t* seeds, dg_denoise_fn denoise,
                        void* user, dg_dtype dtype, void* logits_scratch, int32_t* final_argmax,
                        int32_t* steps_used, uint8_t* stopped, void* stream);

/* The run of dg_run_canvas with its loop state kept on the device
 * ("DiffusionGemma Lab", §2 items 3 and 5; boxwrench.dev Algorithm 1: the
 * loop that stops a canvas once its argmax canvas is stable and its mean
 * entropy is low, or at the step cap). The acceptance kernel itself clears a
 * canvas's active flag when its stop fires, records the steps it used and
 * writes the next step's temperature, so no step waits for the host: the
 * steps are enqueued back to back. Results (final_argmax, steps_used,
 * stopped) equal those of dg_run_canvas for the same seeds and denoiser.
 *   seeds        device uint64 [B] (read by every step; keep it unchanged
 *                until the run's work is done)
 *   final_argmax device int32 [B, L], written
 *   steps_used   device int32 [B], written (1..max_steps)
 *   stopped      device uint8 [B], written: 1 if the adaptive stop fired
 *   check_every  0: enqueue all max_steps steps and return without waiting;
 *                nothing in the call copies memory or synchronises, so a
 *                caller may capture the whole call into a HIP graph and replay
 *                it (steps after every canvas has stopped find no active
 *                canvas and exit at once). k > 0: after every k steps copy the
 *                B active flags to the host, wait for the stream, and end the
 *                loop once no canvas is active; returns after that wait.
 * The denoiser is called once per enqueued step, with the device active flags
 * as they will be when its work runs; logits_scratch, dtype and the callback
 * are as for dg_run_canvas. Errors: as dg_run_canvas, plus DG_ERR_INVALID_ARG
 * for check_every < 0. */
dg_status dg_run_canvas_resident(dg_ctx* ctx, int32_t B, const uint64_t* seeds,
                                 dg_denoise_fn denoise, void* user, dg_dtype dtype,
                                 void* logits_scratch, int32_t* final_argmax, int32_t* steps_used,
                                 uint8_t* stopped, int32_t check_every, void* stream);

/* Callbacks of dg_generate. Like dg_denoise_fn they enqueue work on `stream`
 * and return 0 on success.
 *   dg_block_denoise_fn  writes the logits of step `step` of canvas
 *                        `canvas_index` (arguments otherwise as dg_denoise_fn).
 *   dg_cache_fn          is told, once per canvas and before the next canvas's
 *                        first step, the finished argmax canvases of every
 *                        stream (device int32 [B, L], valid in stream order
 *                        until the next canvas finishes): the extra forward
 *                        pass that appends them to the model's cache. */
typedef int (*dg_block_denoise_fn)(void* user, int32_t canvas_index, int32_t step,
                                   const int32_t* canvas_dev, const uint8_t* active_dev,
                                   void* logits_dev, void* stream);
typedef int (*dg_cache_fn)(void* user, int32_t canvas_index, const int32_t* canvas_dev, void* stream);

/* Block-autoregressive generation of B streams of n_canvases canvases each
 * ("DiffusionGemma Lab", §2, Figure 1: finished canvases chain
 * block-autoregressively; "DiffusionGemma: When the LLM Stops Writing Left to
 * Right", "What DiffusionGemma Actually Is": one canvas at a time, each
 * conditioned on the finished ones; boxwrench.dev "Finding": committed
 * canvases are appended to the encoder's cache canvas by canvas). For
 * k = 0 .. n_canvases-1: the device-resident run of dg_run_canvas_resident
 * for canvas k, whose seed is seeds[c] for k = 0 and otherwise words 0 and 1
 * (low, high) of Philox4x32-10 at counter (k, 0, 0, CANVAS = 4) under
 * key(seeds[c]); its argmax canvas goes to the stream's tokens; then
 * cache_update (if not NULL) is told the finished canvases.
 *   seeds        device uint64 [B]
 *   n_canvases   >= 1, n_canvases * L <= INT32_MAX
 *   tokens       device int32 [B, n_canvases * L], written: stream c's
 *                canvases one after the other
 *   steps_used   device int32 [n_canvases, B], written: steps of canvas k of
 *                stream c at [k * B + c]
 *   stopped      device uint8 [n_canvases, B], written: adaptive stop fired
 *   check_every  as for dg_run_canvas_resident; 0 enqueues every step of every
 *                canvas without waiting (capturable into a HIP graph)
 * Other arguments and errors as dg_run_canvas_resident; a failing
 * cache_update returns DG_ERR_CALLBACK. */
dg_status dg_generate(dg_ctx* ctx, int32_t B, const uint64_t* seeds, int32_t n_canvases,
                      dg_block_denoise_fn denoise, dg_cache_fn cache_update, void* user, dg_dtype dtype,
                      void* logits_scratch, int32_t* tokens, int32_t* steps_used, uint8_t* stopped,
                      int32_t check_every, void* stream);

/* The self-conditioning matmul of the sampling stage (boxwrench.dev,
 * "DiffusionGemma: Parallel Denoising From an Autoregressive Checkpoint",
 * "Finding": a 7.8 M-parameter self-conditioning block feeds the previous
 * step's prediction back; hardware paragraph: the sampling stage runs it with
 * the full-vocabulary softmax, in full precision, over the canvas positions).
 * The pages give no shapes; this library reads it as the expected token
 * embedding under the step's tempered prediction:
 *   out[r, n] = sum_v softmax(z_r / T_c)_v * embed[v, n],  n < d,
 * for the B*L rows r of the logits (c = r / L), at fp32 accuracy on the
 * matrix cores: probabilities and embedding values are fp32, each product is
 * formed from exact three-part bf16 splits of its factors to within about
 * one fp32 rounding, and sums run in fp32 (order unspecified but fixed, so
 * the result is reproducible). With d = 30 at V = 262144 the embedding holds
 * 7,864,320 parameters.
 *   logits, dtype, row_stride  as for dg_canvas_stats, and row_stride times
 *                the element size below 2^27 bytes (V up to about 64 M bf16
 *                or 32 M fp32 ids), else DG_ERR_UNSUPPORTED; ids from V to
 *                row_stride (the padding) never count, whatever they hold
 *   temperature  device float [B], each > 0
 *   argmax       device int32 [B*L]: the row's largest-logit id, as
 *                dg_canvas_stats writes it (the softmax is taken relative to
 *                that logit; another id gives wrong values, never a fault)
 *   embed        device fp32 [V, d], row-major, 4-byte aligned
 *   d            1..31
 *   out          device fp32 [B*L, d], written
 * Uses the context's scratch for partial sums when the batch is small; calls
 * on one context must not overlap. Asynchronous on `stream`. */
dg_status dg_self_condition(dg_ctx* ctx, int32_t B, const void* logits, dg_dtype dtype, int64_t row_stride,
                           const float* temperature, const int32_t* argmax, const float* embed, int32_t d,
                           float* out, void* stream);

/* The sampling stage of one step with the self-conditioning matmul fused
 * after the statistics pass (boxwrench.dev, hardware paragraph: the stage runs
 * the full-vocabulary softmax and the self-conditioning matmul together):
 * dg_canvas_stats, then dg_self_condition on its argmax (selfcond_out
 * [B*L, d] fp32, written for the rows of active canvases only), then
 * dg_accept_renoise. Arguments as for dg_sampler_step and dg_self_condition. */
dg_status dg_sampler_step_selfcond(dg_ctx* ctx, int32_t B, const void* logits, dg_dtype dtype,
                                   int64_t row_stride, const float* temperature, int32_t step,
                                   const uint64_t* seeds, const int32_t* prev_argmax, const uint8_t* active,
                                   const float* embed, int32_t d, float* selfcond_out, const dg_step_out* out,
                                   void* stream);

/* Tokens per forward pass of finished dg_generate streams (boxwrench.dev,
 * "Finding", hardware paragraph: TPF counts the extra forward pass that
 * updates the cache; throughput is TPS = TPF / t_fwd). A stream's forwards
 * are its denoising steps plus one cache update per canvas, and every canvas
 * contributes its L tokens:
 *   tpf[c]   = n_canvases * L / (sum_k steps_used[k * B + c] + n_canvases)
 *   tpf_all  = n_canvases * B * L / (sum over streams of those forwards)
 *   steps_used  host int32 [n_canvases, B], each >= 0
 *   tpf         host double [B] or NULL;  tpf_all: host double or NULL
 * Host arithmetic only; no context needed. */
dg_status dg_tokens_per_forward(const int32_t* steps_used, int32_t n_canvases, int32_t B,
                                int32_t canvas_len, double* tpf, double* tpf_all);

/* LM-head projection feeding the sampler: the pages' sampling stage runs a
 * full-vocabulary softmax over the 256 canvas positions (boxwrench.dev,
 * "DiffusionGemma: Parallel Denoising From an Autoregressive Checkpoint", the
 * hardware breakdown of one denoising step); its logits are the product of the
 * decoder's last hidden states with the LM-head weights:
 *   logits[r, v] = sum_k hidden[r, k] * weight[k, v]
 * computed from bf16 operands with fp32 accumulation on the matrix cores
 * (summation order unspecified) and stored as fp32.
 *   rows        >= 1
 *   hidden      device bf16 [rows, hidden_dim], row-major (K contiguous)
 *   weight      device bf16 [hidden_dim, V], row-major (V contiguous), V the
 *               context's vocab
 *   hidden_dim  K: a positive multiple of 64      (else DG_ERR_UNSUPPORTED)
 *   logits      device fp32 [rows, ld_logits], written in columns [0, V)
 *   ld_logits   >= V, a multiple of 4
 * V must be a multiple of 8 and each of rows*K*2 and K*V*2 bytes at most
 * 0x7FFF0000 (DG_ERR_UNSUPPORTED otherwise); the three arrays must be 16-byte
 * aligned. Asynchronous on `stream`. */
dg_status dg_lmhead_logits(dg_ctx* ctx, int32_t rows, const void* hidden, const void* weight,
                           int32_t hidden_dim, float* logits, int64_t ld_logits, void* stream);

/* Device workspace, in bytes, that dg_lmhead_sampler_step needs for B
 * canvases (1 <= B <= max_batch): 40 * B * L * 16 * ceil(V / 4096) + 4 * B * L.
 *   bytes   host int64 out */
dg_status dg_lmhead_workspace_bytes(const dg_ctx* ctx, int32_t B, int64_t* bytes);

/* One sampler step of B canvases whose logits come from the LM head, with the
 * logits never stored: the product of dg_lmhead_logits (the same fp32 values
 * bit for bit) feeds the statistics of dg_sampler_step inside the product's
 * own epilogue. Every 256 x 256 tile of the product holds four whole blocks of
 * the sampler's two-level Gumbel-max protocol, so the tile reduces each of its
 * rows to one partial (maximum and its first id, the entropy sums, its best
 * block's score and the in-block draw of that block; "DiffusionGemma Lab",
 * §2 items 2 and 5); a merge of every row's partials gives the entropy,
 * argmax and sample, and the acceptance of dg_sampler_step follows.
 * Argmax and acceptance inputs are those of dg_sampler_step on the
 * dg_lmhead_logits product: the argmax is identical, the entropy agrees to
 * fp32 rounding of the sums, and the sample is identical except where two
 * perturbed scores lie within fp32 rounding of each other.
 *   workspace        device, 16-byte aligned, at least
 *                    dg_lmhead_workspace_bytes(ctx, B) bytes (else
 *                    DG_ERR_INVALID_ARG); its contents are overwritten
 *   temperature      device float [B]
 *   step             the step index of every canvas when `steps` is NULL
 *   steps            device int32 [B] or NULL: canvas c draws its random
 *                    numbers for step steps[c] (values >= 0, not checked), so
 *                    canvases at different points of their schedules share
 *                    one call
 *   active           device uint8 [B] or NULL: as for dg_sampler_step; tiles
 *                    whose rows all lie in inactive canvases are not computed
 * hidden, weight and hidden_dim are those of dg_lmhead_logits (the same shape
 * limits); seeds, prev_argmax and out those of dg_sampler_step. Products that
 * overflow fp32 (an infinite logit) give unspecified statistics. Asynchronous
 * on `stream`. */
dg_status dg_lmhead_sampler_step(dg_ctx* ctx, int32_t B, const void* hidden, const void* weight,
                                 int32_t hidden_dim, void* workspace, int64_t workspace_bytes,
                                 const float* temperature, int32_t step, const int32_t* steps,
                                 const uint64_t* seeds, const int32_t* prev_argmax, const uint8_t* active,
                                 const dg_step_out* out, void* stream);

/* dg_sampler_step for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * context, no allocation of any kind. The step's intermediate statistics and
 * split-row partials live in a static device array (about 200 KiB) that each
 * GPU the library runs on holds until the process ends; its address is looked
 * up once per device on the first call made with that device current.
 *   params   host; the step's settings, as for dg_create (checked the same way)
 *   B        1 .. 16384 / params->canvas_len (at most 16384 rows): larger
 *            batches return DG_ERR_INVALID_ARG without writing anything
 * The other arguments and every result are those of dg_sampler_step on the
 * current device; the results equal dg_sampler_step's bit for bit. Every call
 * on one GPU shares that GPU's array, and a call clears what it needs cleared,
 * so calls that overlap on one GPU (concurrent streams) race: serialise them.
 * Errors are reported through dg_last_error(NULL). */
dg_status dg_sampler_step_noalloc(const dg_params* params, int32_t B, const void* logits, dg_dtype dtype,
                                  int64_t row_stride, const float* temperature, int32_t step,
                                  const uint64_t* seeds, const int32_t* prev_argmax, const uint8_t* active,
                                  const dg_step_out* out, void* stream);

/* Library version string. */
const char* dg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DG_CANVAS_H */
