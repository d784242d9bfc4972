"""Pins of the oracle's LM-head projection (oracle.lmhead) against things other
than itself: pure-Python dot products, exact rational arithmetic, one-hot
weights, exact power-of-two scaling, and the closed form of zero hidden states
(uniform logits: H = ln V everywhere, exactly one commit)."""
from fractions import Fraction

import numpy as np
import torch

from canvas_sampler_amd import synth
from oracle import lmhead as OL


def _bf16_values(t):
    return t.to(torch.float32).numpy()


def _operands(rows, k, vocab, seed=7):
    h, w = synth.lmhead_operands(seed, rows, k, vocab)
    return _bf16_values(h), _bf16_values(w)


def test_pure_python_dot_products():
    h, w = _operands(5, 24, 11)
    z = OL.logits(h, w, col_chunk=4)
    for r in range(h.shape[0]):
        for v in range(w.shape[1]):
            acc = 0.0
            for k in range(h.shape[1]):
                acc += float(h[r, k]) * float(w[k, v])
            assert abs(z[r, v] - acc) <= 1e-12 * (1 + abs(acc))


def test_exact_rational_sum_within_fp64_bound():
    h, w = _operands(3, 256, 9, seed=11)
    z = OL.logits(h, w)
    for r in range(h.shape[0]):
        for v in range(w.shape[1]):
            exact = sum(Fraction(float(h[r, k])) * Fraction(float(w[k, v])) for k in range(h.shape[1]))
            mag = sum(abs(float(h[r, k]) * float(w[k, v])) for k in range(h.shape[1]))
            assert abs(Fraction(z[r, v]) - exact) <= Fraction(h.shape[1] * mag) / 2**53


def test_one_hot_weight_columns_select_hidden_columns():
    rng = np.random.default_rng(3)
    k, vocab = 64, 40
    h, _ = _operands(7, k, vocab)
    pick = rng.integers(0, k, size=vocab)
    w = np.zeros((k, vocab), dtype=np.float32)
    w[pick, np.arange(vocab)] = 1.0
    z = OL.logits(h, w, col_chunk=16)
    assert np.array_equal(z, h[:, pick].astype(np.float64))


def test_power_of_two_scaling_is_exact():
    h, w = _operands(4, 128, 33)
    z = OL.logits(h, w)
    assert np.array_equal(OL.logits(h, w * 4.0), 4.0 * z)
    assert np.array_equal(OL.logits(h * 0.5, w), 0.5 * z)


def test_transposed_operand_shapes_checked():
    h, w = _operands(2, 64, 8)
    try:
        OL.logits(h, w[:32])
    except ValueError:
        return
    raise AssertionError("mismatched K accepted")


def test_zero_hidden_states_give_uniform_canvas():
    L, k, vocab = 16, 64, 4096
    _, w = _operands(1, k, vocab)
    out = OL.step(np.zeros((L, k), dtype=np.float32), w, np.float32(0.8), 0, 0)
    assert np.all(out["logits"] == 0.0)
    assert np.allclose(out["entropy"], np.log(vocab), atol=1e-12)
    assert out["n_accept"] == 1 and out["accept"][0] and out["accept"].sum() == 1
    assert not out["stop"]
