"""Oracle of the canvas sampler: a plain, slow, fp64 CPU implementation of what
the HIP path computes, written from the pages' description of the sampler.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
CPU-baseline leg may import it. The product path (canvas_sampler_amd and the
HIP library) never calls it, and the two share no code.

Pins (tests/test_oracle_*.py, run with -m "not gpu"):
  philox.philox4x32_10   Random123 known-answer vectors; PyTorch ATen engine
  philox.uniform_open01  exact endpoints, chi-square uniformity
  sampler.temperature    numpy.linspace in fp32; clamp; single-step schedule
  sampler.entropy        closed forms (ln V, 0, ln k), scipy.stats.entropy,
                         6.91 nats at V = 1000 ("DiffusionGemma Lab" EXP A)
  sampler.argmax_raw     planted maxima and ties, brute-force loop
  sampler.block_*        brute-force membership loop, partition of [0, V)
  sampler.sample_*       chi-square against softmax; planted dominant id;
                         two-level vs per-element agreement in distribution
  sampler.accept         brute-force subset enumeration (L <= 12); equal-
                         entropy closed form; >= 1 commit; monotone in b
  sampler.uniform_tokens chi-square; top-bits formula for power-of-two V
  sampler.stop_test      truth table
  sampler.step / run     constant canvas (ln V, 1 commit, no stop); one-hot
                         canvas (H = 0, all commit, stops at the 2nd step);
                         low-confidence canvas (1 commit/step, 48-step cap);
                         trend directions of "DiffusionGemma Lab" EXP B.
  lmhead.logits          pure-Python dot products; exact rational sums within
                         K * 2^-53; one-hot weight columns select hidden
                         columns exactly; power-of-two scaling is exact
  lmhead.step            zero hidden states give uniform logits: H = ln V at
                         every position and exactly one commit
  selfcond.self_condition one-hot rows select an embedding row; uniform rows
                         average the embedding; a column of ones gives total
                         probability 1; indicator columns equal brute-force
                         probability sums; an index column gives the closed-form
                         truncated geometric mean; linear in E, invariant to
                         logit shifts (tests/test_oracle_selfcond.py)
  blockar.canvas_seed    Philox words of the canvas counter (known-answer
                         vectors via philox); blockar.tokens_per_forward and
                         tokens_per_second: the pages' own TPS arithmetic
                         (tests/golden/tps_worked_example_boxwrench.txt);
  blockar.generate       a never-confident stream runs every canvas to the
                         cap, a certain stream stops every canvas at step two
                         and chains its targets (tests/test_oracle_blockar.py)
  parallel.steps         equal, key for key, to sampler.step on the same rows
                         (it only spreads sampler.row_statistics over threads)
No function is parity-unpinned. The bit-level choice of the random protocol
(block partition, grouping of the block words) is pinned only by agreement
of the two independent implementations; the pages fix the sample in
distribution only, which the chi-square tests pin.
"""
from . import blockar, lmhead, parallel, philox, sampler, selfcond  # noqa: F401
