// Host-side paths of the C ABI (include/dg_canvas.h) that need no GPU:
// parameter validation and its messages, the temperature schedule, the
// tokens-per-forward accounting, NULL handles, and context creation on a
// machine without a usable device. Built with address and undefined-behaviour
// sanitizers on the host code by tests/test_library_host.py; exits non-zero
// on the first unexpected result.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "dg_canvas.h"

static int failures = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                        \
    }                                                                    \
  } while (0)

static bool names(const char* msg, const char* what) { return msg && std::strstr(msg, what) != nullptr; }

int main() {
  dg_params p;
  EXPECT(dg_params_default(&p) == DG_OK);
  EXPECT(p.canvas_len == 256 && p.vocab == 262144 && p.max_steps == 48);
  EXPECT(dg_params_check(&p) == DG_OK);
  EXPECT(dg_params_default(nullptr) == DG_ERR_INVALID_ARG);

  // every field out of range is named in the message
  struct Bad {
    const char* field;
    void (*set)(dg_params*);
  } bad[] = {
      {"canvas_len", [](dg_params* q) { q->canvas_len = 0; }},
      {"canvas_len", [](dg_params* q) { q->canvas_len = 257; }},
      {"vocab", [](dg_params* q) { q->vocab = 1; }},
      {"entropy_bound", [](dg_params* q) { q->entropy_bound = -0.1f; }},
      {"entropy_bound", [](dg_params* q) { q->entropy_bound = NAN; }},
      {"temp_start", [](dg_params* q) { q->temp_start = 0.0f; }},
      {"temp_end", [](dg_params* q) { q->temp_end = INFINITY; }},
      {"temp_steps", [](dg_params* q) { q->temp_steps = 0; }},
      {"max_steps", [](dg_params* q) { q->max_steps = 0; }},
      {"stop_mean_entropy", [](dg_params* q) { q->stop_mean_entropy = -1.0f; }},
  };
  for (const Bad& b : bad) {
    dg_params q;
    dg_params_default(&q);
    b.set(&q);
    EXPECT(dg_params_check(&q) == DG_ERR_INVALID_ARG);
    EXPECT(names(dg_last_error(nullptr), b.field));
  }

  // the schedule stays between its end points and clamps after its last step
  for (int S = 1; S <= 64; ++S) {
    dg_params q;
    dg_params_default(&q);
    q.temp_steps = S;
    for (int s = 0; s < 100; ++s) {
      float t = -1.0f;
      EXPECT(dg_temperature(&q, s, &t) == DG_OK);
      EXPECT(std::isfinite(t) && t >= 0.4f && t <= 0.8f);
      if (s >= S - 1) {
        float last = -1.0f;
        dg_temperature(&q, S - 1, &last);
        EXPECT(t == last);
      }
    }
  }
  float t = 0.0f;
  EXPECT(dg_temperature(&p, -1, &t) == DG_ERR_INVALID_ARG);
  EXPECT(dg_temperature(&p, 0, nullptr) == DG_ERR_INVALID_ARG);

  // tokens per forward
  std::vector<int32_t> steps = {48, 2, 10, 7, 1, 48};  // [3 canvases, 2 streams]
  double per[2] = {0, 0}, all = 0;
  EXPECT(dg_tokens_per_forward(steps.data(), 3, 2, 256, per, &all) == DG_OK);
  EXPECT(std::fabs(per[0] - 3.0 * 256 / (48 + 10 + 1 + 3)) < 1e-12);
  EXPECT(std::fabs(per[1] - 3.0 * 256 / (2 + 7 + 48 + 3)) < 1e-12);
  EXPECT(std::fabs(all - 6.0 * 256 / (62 + 60)) < 1e-12);
  steps[3] = -1;
  EXPECT(dg_tokens_per_forward(steps.data(), 3, 2, 256, per, &all) == DG_ERR_INVALID_ARG);
  EXPECT(names(dg_last_error(nullptr), "steps_used[3]"));
  EXPECT(dg_tokens_per_forward(nullptr, 3, 2, 256, nullptr, nullptr) == DG_ERR_INVALID_ARG);

  // NULL handles are rejected by every entry point that takes one
  EXPECT(dg_destroy(nullptr) == DG_OK);
  EXPECT(dg_get_params(nullptr, &p) == DG_ERR_INVALID_ARG);
  EXPECT(dg_set_stats_split(nullptr, 1) == DG_ERR_INVALID_ARG);
  EXPECT(dg_canvas_init(nullptr, 1, nullptr, nullptr, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_canvas_stats(nullptr, 1, nullptr, DG_DTYPE_BF16, 0, nullptr, 0, nullptr, nullptr, nullptr, nullptr,
                         nullptr, nullptr) == DG_ERR_INVALID_ARG);
  dg_step_out o;
  std::memset(&o, 0, sizeof(o));
  EXPECT(dg_sampler_step(nullptr, 1, nullptr, DG_DTYPE_BF16, 0, nullptr, 0, nullptr, nullptr, nullptr, &o,
                         nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_accept_renoise(nullptr, 1, nullptr, nullptr, nullptr, 0, nullptr, nullptr, nullptr, &o, nullptr) ==
         DG_ERR_INVALID_ARG);
  EXPECT(dg_run_canvas(nullptr, 1, nullptr, nullptr, nullptr, DG_DTYPE_BF16, nullptr, nullptr, nullptr, nullptr,
                       nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_run_canvas_resident(nullptr, 1, nullptr, nullptr, nullptr, DG_DTYPE_BF16, nullptr, nullptr, nullptr,
                                nullptr, 0, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_generate(nullptr, 1, nullptr, 1, nullptr, nullptr, nullptr, DG_DTYPE_BF16, nullptr, nullptr, nullptr,
                     nullptr, 0, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_self_condition(nullptr, 1, nullptr, DG_DTYPE_BF16, 0, nullptr, nullptr, nullptr, 30, nullptr,
                           nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_sampler_step_selfcond(nullptr, 1, nullptr, DG_DTYPE_BF16, 0, nullptr, 0, nullptr, nullptr, nullptr,
                                  nullptr, 30, nullptr, &o, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(dg_lmhead_logits(nullptr, 1, nullptr, nullptr, 64, nullptr, 0, nullptr) == DG_ERR_INVALID_ARG);
  EXPECT(names(dg_last_error(nullptr), "ctx"));

  // creation: invalid arguments first, then the device (none is usable here)
  dg_ctx* ctx = reinterpret_cast<dg_ctx*>(0x1);
  EXPECT(dg_create(&ctx, 0, 0, &p) == DG_ERR_INVALID_ARG && ctx == nullptr);
  EXPECT(names(dg_last_error(nullptr), "max_batch"));
  const dg_status st = dg_create(&ctx, 0, 1, &p);
  if (st == DG_OK) {
    EXPECT(dg_destroy(ctx) == DG_OK);  // a device was present after all
  } else {
    EXPECT(st == DG_ERR_DEVICE && ctx == nullptr);
  }
  EXPECT(dg_version() != nullptr && std::strlen(dg_version()) > 0);

  if (failures) std::fprintf(stderr, "%d unexpected results\n", failures);
  else std::printf("host ABI checks passed\n");
  return failures ? 1 : 0;
}
