// Internal launch interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// Partial result of the statistics pass over part of a row (40 bytes): of a
// wave, of a workgroup, or of a split of a row over several workgroups.
//   s, w     sums of 2^t and t*2^t, t = z*c - ref with c = log2(e)/T and ref
//            an fp32 value at most the part's max z*c (-inf: nothing finite)
//   ref      that reference
//   m        largest raw logit; argmax = lowest id attaining it
//   best     largest block score (log2 units), bestj its block, and sample
//            the in-block Gumbel-max draw of that block
struct RowPartial {
  double s;
  double w;
  float ref;
  float m;
  int32_t argmax;
  float best;
  int32_t bestj;
  int32_t sample;
};

struct AcceptArgs {
  const float* entropy;
  const int32_t* argmax;
  const int32_t* sample;
  const uint64_t* seeds;
  const int32_t* prev_argmax;  // may be null
  const uint8_t* active;       // may be null
  int32_t step;
  const int32_t* steps;        // may be null: per-canvas step, else `step`
  int32_t canvas_len;
  int32_t vocab;
  float bound;
  float stop_mean_entropy;
  int32_t* canvas_out;
  int32_t* argmax_out;         // may be null: copy of argmax
  int32_t* sample_out;         // may be null: copy of sample
  float* entropy_out;          // may be null: copy of entropy
  uint8_t* accept_out;         // may be null
  int32_t* n_accept_out;       // may be null
  float* mean_entropy_out;     // may be null
  uint8_t* stop_out;           // may be null
  // Loop state of a device-resident run (all null outside one): a canvas
  // that runs this step records step + 1 in run_steps_used and the next
  // step's temperature in run_temperature; when its stop fires it sets
  // run_stopped and clears run_active (the same flags as `active`).
  uint8_t* run_active;
  int32_t* run_steps_used;
  uint8_t* run_stopped;
  float* run_temperature;
  float run_next_temperature;
};

struct StatsArgs {
  const void* logits;
  int64_t row_stride;      // elements
  int32_t vocab;
  int32_t canvas_len;
  int32_t rows;            // B * L
  int32_t nsplit;          // workgroups per row
  const float* temperature;
  const uint64_t* seeds;
  int32_t step;
  const int32_t* steps;    // may be null: per-canvas step, else `step`
  const uint8_t* active;   // may be null
  float* entropy;
  int32_t* argmax;
  int32_t* sample;
  RowPartial* partials;    // [rows * nsplit] when nsplit > 1: merged by launch_partials_merge
  int32_t row_grid;        // > 0: a persistent grid of this many workgroups loops over the rows
};

// LM-head projection: logits[r, v] = sum_k hidden[r, k] * weight[k, v].
struct GemmArgs {
  const void* hidden;      // bf16 [rows, hidden_dim]
  const void* weight;      // bf16 [hidden_dim, vocab]
  float* logits;           // fp32 [rows, ld_logits] (the product alone)
  int64_t ld_logits;
  int32_t rows;
  int32_t hidden_dim;      // multiple of 64
  int32_t vocab;           // multiple of 8
  // The product with the statistics epilogue (logits never stored): each
  // 256 x 256 tile holds four whole blocks of the sampling protocol and
  // writes one RowPartial per row into partials[row * ntiles + tile].
  int32_t canvas_len;
  const float* temperature;   // [rows / canvas_len]
  const uint64_t* seeds;
  int32_t step;
  const int32_t* steps;       // may be null: per-canvas step, else `step`
  const uint8_t* active;      // may be null: tiles whose rows all lie in inactive canvases are skipped
  RowPartial* partials;       // [rows, ntiles]
  uint32_t* hint;             // [rows]: best block score so far (order-preserving bits), zero at launch
  int32_t ntiles;             // tiles per row: 16 * ceil(vocab / 4096)
};

// Self-conditioning matmul: out[r, n] = sum_v softmax(z_r / T)_v E[v, n].
struct SelfCondArgs {
  const void* logits;      // [rows, row_stride], bf16 or fp32
  int64_t row_stride;      // elements
  int32_t vocab;
  int32_t canvas_len;      // rows of one canvas (temperature index = row / canvas_len)
  int32_t rows;
  const float* temperature;  // [rows / canvas_len]
  const int32_t* argmax;   // [rows]: id of each row's largest logit
  const uint8_t* active;   // [rows / canvas_len] or null: rows of inactive canvases are skipped
  const float* embed;      // fp32 [vocab, d]
  int32_t d;               // 1..31
  float* out;              // fp32 [rows, d]
  int32_t nslice;          // vocabulary slices per row tile
  int32_t kslice;          // ids per slice (a multiple of 64)
  int32_t rows_pad;        // rows rounded up to the row tile
  float* partials;         // [nslice, rows_pad, 32] when nslice > 1
};

constexpr int kScThreads = 512;          // 8 waves x 32 rows
constexpr int kScRowTile = 256;
// Slices are cut so that tiles * slices <= this. At 256 rows x 262144 ids:
// 256 workgroups (slices of 1024 ids) 57 us, 512 61 us, 384 68 us, 1024 68 us.
constexpr int kScTargetWorkgroups = 256;

// Vocabulary slices for `rows` rows: one per row tile when the tiles alone
// fill the target, else about kScTargetWorkgroups / tiles slices.
void choose_self_cond_slices(int32_t rows, int32_t vocab, int32_t* nslice, int32_t* kslice);
hipError_t launch_self_cond(const SelfCondArgs& a, bool bf16, hipStream_t stream);

constexpr int kGemmThreads = 512;

constexpr int kStatsThreads = 512;   // 8 waves: one workgroup streams a whole row
constexpr int kAcceptThreads = 256;

// Chooses the number of workgroups per row for `rows` rows of `vocab` ids.
int32_t choose_nsplit(int32_t rows, int32_t vocab);
// Workgroups of the persistent row loop for this launch, or 0 for one
// workgroup per row (or split).
int32_t stats_row_grid(int32_t rows, int32_t vocab, int32_t nsplit, bool has_active, int32_t cu_count);

hipError_t launch_canvas_stats(const StatsArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_accept_renoise(const AcceptArgs& a, int32_t batch, hipStream_t stream);
hipError_t launch_lmhead_gemm(const GemmArgs& g, hipStream_t stream);
// The product with the statistics epilogue, then the merge of each row's tile
// partials into a.entropy / a.argmax / a.sample (a: rows, vocab, canvas_len,
// active as for the statistics pass). Tiles per row for `vocab`:
int32_t lmhead_stats_tiles(int32_t vocab);
hipError_t launch_lmhead_stats(const GemmArgs& g, hipStream_t stream);
hipError_t launch_partials_merge(const StatsArgs& a, const RowPartial* partials, int32_t nparts,
                                 hipStream_t stream);
// Start of a device-resident run: every canvas active, no steps used, not
// stopped, temperature t0.
hipError_t launch_run_state_init(int32_t batch, uint8_t* active, int32_t* steps_used,
                                 uint8_t* stopped, float* temperature, float t0, hipStream_t stream);
// Seeds of canvas k of B block-autoregressive streams: out[c] = seeds[c] for
// k = 0, else words 0 and 1 of Philox4x32-10 at counter (k, 0, 0, CANVAS)
// under key(seeds[c]).
hipError_t launch_canvas_seeds(const uint64_t* seeds, int32_t batch, int32_t k, uint64_t* out,
                               hipStream_t stream);
// tokens[c * ld + offset + l] = canvas[c * canvas_len + l] for c < batch, l < canvas_len.
hipError_t launch_place_canvas(const int32_t* canvas, int32_t batch, int32_t canvas_len, int32_t* tokens,
                               int64_t ld, int64_t offset, hipStream_t stream);
// p[0..n) = value, as a kernel (so that a captured graph holds no memset node).
hipError_t launch_fill_u32(uint32_t* p, int32_t n, uint32_t value, hipStream_t stream);
hipError_t launch_canvas_init(const uint64_t* seeds, int32_t batch, int32_t canvas_len,
                              int32_t vocab, int32_t* canvas, hipStream_t stream);

}  // namespace dg
