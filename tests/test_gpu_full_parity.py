"""Every row of every step of the four sampler workloads against the oracle, at
full size (256 positions per canvas; V = 4096 fp32 for the single margin step,
V = 262144 for the rest), through the C ABI.

Each test runs the workload's canvases to their adaptive stop (or the
48-step cap) twice on the GPU: stepped from Python with every output read
back, and through the library's own loop (dg_run_canvas). The oracle runs on
the same logits bits, all rows, every step (tests/full_parity.py). Steps used,
stop flags and final argmax canvases must be equal; per-step differences are
allowed only at counted near-ties, which each test prints.
"""
import math

import numpy as np
import pytest
import torch

from canvas_sampler_amd import synth

from full_parity import sharpening_writer, trajectory
from gpu_util import gpu, require_gpu

pytestmark = [gpu, pytest.mark.timeout(900)]

L, V_FULL = 256, 262144


def test_c1_margin_step_all_rows():
    # one canvas, V = 4096 fp32: N(0,1) plus m ~ U[0, 12] at a uniform target,
    # T = 0.8, seed 0; one step (the cap), no stop possible at step 0
    require_gpu()
    V = 4096

    def write(step, out):
        synth.margin_logits(1001, L, V, m_max=12.0, dtype=torch.float32, device="cuda", out=out)

    tally, runs, commits = trajectory("C1", L, V, [0], write, torch.float32, cap=1)
    assert runs[0][:2] == (1, False)
    assert commits[0][0] >= 1
    tally.report()


def test_c2_single_canvas_full_vocab_trajectory():
    # the benchmark canvas: B = 1, 256 x 262144 bf16 sharpening logits
    # (m0 ~ U[0, 6], growth 1.5 per step), T 0.8 -> 0.4 over 16 steps, b = 0.1,
    # adaptive stop, cap 48
    require_gpu()
    write = sharpening_writer([1002], L, V_FULL, 6.0, torch.bfloat16)
    tally, runs, commits = trajectory("C2", L, V_FULL, [0], write, torch.bfloat16, temp_steps=16)
    assert runs[0][1], "the sharpening canvas must stop before the cap"
    assert 2 <= runs[0][0] < 48
    assert tally.trajectories_equal == 1
    print("C2 commits per step", commits[0])
    tally.report()


def test_c3_sixteen_canvases_full_vocab_trajectories():
    # 16 independent canvases, 256 x 262144 bf16 each, per-canvas generator
    # seeds (1003 << 32) | c with m0 ~ U[0, 8] and sampler seeds c, the same
    # schedule as the single canvas (0.8 -> 0.4 over 16 steps), adaptive stop
    # per canvas (stopped canvases leave the batch), cap 48
    require_gpu()
    n = 16
    write = sharpening_writer([(1003 << 32) | c for c in range(n)], L, V_FULL, 8.0, torch.bfloat16)
    tally, runs, commits = trajectory("C3", L, V_FULL, list(range(n)), write, torch.bfloat16, temp_steps=16)
    assert all(r[1] for r in runs), "every sharpening canvas must stop before the cap"
    assert tally.trajectories_equal == n
    print("C3 steps per canvas", [r[0] for r in runs])
    tally.report()


def test_c4_low_confidence_fp32_to_the_cap():
    # untrained-model stand-in: iid N(0, 0.05) fp32 logits at V = 262144, fresh
    # each step, default schedule (0.8 -> 0.4 over 48 steps): exactly one
    # commit per step and no stop before the 48-step cap ("DiffusionGemma Lab"
    # EXP A); the mean entropy follows ln V - sigma^2 / (2 T^2) to first order
    require_gpu()

    def write(step, out):
        synth.iid_normal_logits(1004, step, L, V_FULL, variance=0.05, dtype=torch.float32, device="cuda", out=out)

    mean_h = {}

    def on_step(s, c, g, o):
        mean_h[s] = float(np.mean(np.asarray(g["entropy"], dtype=np.float64)))

    tally, runs, commits = trajectory("C4", L, V_FULL, [0], write, torch.float32, temp_steps=48,
                                      on_step=on_step)
    assert runs[0][:2] == (48, False)
    assert commits[0] == [1] * 48
    from canvas_sampler_amd import binding as B
    params = B.params_default(canvas_len=L, vocab=V_FULL)
    for s, mh in mean_h.items():
        t = B.dg_temperature(params, s)
        assert abs(mh - (math.log(V_FULL) - 0.05 / (2 * t * t))) < 0.03
    tally.report()
