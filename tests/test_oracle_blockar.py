"""Pins of the block-autoregressive driver oracle (oracle/blockar.py): closed
forms of its step and forward counts, a brute-force chain of targets, the
pages' own TPS arithmetic, and the seed derivation's Philox words."""
import os

import numpy as np
import pytest
import torch

from canvas_sampler_amd import synth
from oracle import blockar as BA
from oracle import philox as OP

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_canvas_seeds():
    for s in (0, 1, 2**63 + 5, 2**64 - 1):
        assert BA.canvas_seed(s, 0) == s & (2**64 - 1)
    seen = set()
    for s in (0, 1):
        for k in range(200):
            seen.add(BA.canvas_seed(s, k))
    assert len(seen) == 400
    # canvas k >= 1: the first two words of the (known-answer pinned) Philox
    # call for counter (k, 0, 0, CANVAS) under the stream's key
    w = OP.philox4x32_10(3, 0, 0, OP.TAG_CANVAS, 0x89ABCDEF, 0x01234567)
    assert BA.canvas_seed(0x0123456789ABCDEF, 3) == int(w[0]) + (int(w[1]) << 32)
    assert OP.TAG_CANVAS not in (OP.TAG_INIT, OP.TAG_BLOCK, OP.TAG_ELEM, OP.TAG_RENOISE)


def test_pages_tps_arithmetic():
    path = os.path.join(ROOT, "tests", "golden", "tps_worked_example_boxwrench.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    for tpf, t_fwd, printed in rows:
        assert round(BA.tokens_per_second(float(tpf), float(t_fwd))) == int(printed)


def _zeros(L, V):
    return lambda k, s, canvas: np.zeros((L, V))


def test_never_confident_stream_runs_every_canvas_to_the_cap():
    # all-zero logits: every entropy is ln V, one commit per step, the mean
    # entropy never falls below 0.005, so each canvas uses all 48 steps; its
    # argmax canvas is id 0 everywhere (lowest id among equal logits)
    L, V, n = 8, 64, 3
    told = []
    tokens, steps, stopped = BA.generate(_zeros(L, V), lambda k, t: told.append((k, t.copy())),
                                         seed=5, n_canvases=n, canvas_len=L, vocab=V, n_sched=16)
    assert steps == [48] * n and stopped == [False] * n
    assert np.array_equal(tokens, np.zeros(n * L))
    assert [k for k, _ in told] == list(range(n))
    assert BA.forwards(steps) == 3 * 48 + 3
    assert BA.tokens_per_forward(steps, L) == pytest.approx(n * L / (3 * 48 + 3), rel=1e-15)


def _certain_denoiser(gen, L, V, confident=lambda k: True):
    """Logits 0 with +1000 at canvas k's chained targets (confident canvases),
    else all 0; targets of canvas k+1 come from the canvas told to the cache."""
    state = {"target": {0: synth.chained_targets(gen, 0, None, L, V)[0].numpy()}}

    def denoise(k, s, canvas):
        z = np.zeros((L, V))
        if confident(k):
            z[np.arange(L), state["target"][k]] = 1000.0
        return z

    def cache(k, tokens):
        state["target"][k + 1] = synth.chained_targets(gen, k + 1, torch.as_tensor(tokens), L, V)[0].numpy()

    return denoise, cache


def test_certain_stream_stops_every_canvas_at_step_two_and_chains_targets():
    # one-hot logits (margin 1000): zero entropy, argmax = sample = target at
    # every position, so step 0 commits the whole canvas and step 1 (stable
    # argmax, mean entropy 0) stops it; each canvas's output is its targets,
    # and the targets of canvas k+1 continue canvas k's output
    L, V, n, gen = 16, 256, 4, 77
    den, cache = _certain_denoiser(gen, L, V)
    tokens, steps, stopped = BA.generate(den, cache, seed=9, n_canvases=n, canvas_len=L, vocab=V,
                                         n_sched=16)
    assert steps == [2] * n and stopped == [True] * n
    chain = [synth.chained_targets(gen, 0, None, L, V)[0].numpy()]
    for k in range(1, n):
        chain.append(synth.chained_targets(gen, k, torch.as_tensor(chain[-1]), L, V)[0].numpy())
    assert np.array_equal(tokens, np.concatenate(chain))
    # canvas k+1 continues canvas k: target_l = (prev_{l+1} + shift) mod V
    for k in range(1, n):
        d = (chain[k] - np.roll(chain[k - 1], -1)) % V
        assert len(set(d.tolist())) == 1 and d[0] != 0
    assert BA.tokens_per_forward(steps, L) == pytest.approx(n * L / (2 * n + n), rel=1e-15)


def test_mixed_stream_counts_each_canvas():
    L, V, gen = 8, 128, 3
    den, cache = _certain_denoiser(gen, L, V, confident=lambda k: k == 1)
    tokens, steps, stopped = BA.generate(den, cache, seed=0, n_canvases=3, canvas_len=L, vocab=V,
                                         n_sched=16)
    assert steps == [48, 2, 48] and stopped == [False, True, False]
    assert BA.tokens_per_forward(steps, L) == pytest.approx(3 * L / (98 + 3), rel=1e-15)


def test_later_canvases_draw_from_their_own_seeds():
    # with a denoiser that ignores the canvas index, canvas k of the stream is
    # the single-canvas run with seed canvas_seed(seed, k)
    from oracle import sampler as O
    L, V = 8, 64
    rng = np.random.default_rng(4)
    z = rng.normal(size=(L, V)) * 0.3

    tokens, steps, _ = BA.generate(lambda k, s, c: z, None, seed=11, n_canvases=3, canvas_len=L,
                                   vocab=V, n_sched=16, max_steps=6)
    for k in range(3):
        ref, n, _, _ = O.run(lambda s, c: z, BA.canvas_seed(11, k), L, V, n_sched=16, max_steps=6)
        assert np.array_equal(tokens[k * L:(k + 1) * L], ref) and steps[k] == n
    inits = [O.init_canvas(BA.canvas_seed(11, k), L, V) for k in range(3)]
    assert not np.array_equal(inits[0], inits[1]) and not np.array_equal(inits[1], inits[2])
