"""Pins of the oracle's Philox4x32-10 and uniform map against sources other
than itself: the Random123 known-answer vectors and PyTorch's ATen engine."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
import scipy.stats

from oracle import philox

HERE = os.path.dirname(os.path.abspath(__file__))


def _kat_cases(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            rows.append([int(t, 16) for t in line.split()])
    return rows


def test_known_answer_vectors(golden_dir):
    cases = _kat_cases(golden_dir)
    assert len(cases) == 3
    for c in cases:
        out = philox.philox4x32_10(*c[:6])
        assert [int(w) for w in out] == c[6:]


def test_vectorised_matches_scalar_calls():
    rng = np.random.default_rng(5)
    ctr = rng.integers(0, 2**32, size=(4, 50), dtype=np.uint64)
    key = rng.integers(0, 2**32, size=(2, 50), dtype=np.uint64)
    vec = philox.philox4x32_10(*ctr, *key)
    for i in range(50):
        one = philox.philox4x32_10(*[int(x[i]) for x in ctr], *[int(k[i]) for k in key])
        assert [int(w) for w in one] == [int(w[i]) for w in vec]


def _aten_binary():
    import torch
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    if shutil.which("g++") is None or not os.path.exists(
            os.path.join(inc, "ATen", "core", "PhiloxRNGEngine.h")):
        pytest.skip("g++ or the ATen Philox header is not available")
    out = os.path.join(tempfile.mkdtemp(prefix="philox_aten_"), "philox_aten_ref")
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", inc,
                    os.path.join(HERE, "philox_aten_ref.cpp"), "-o", out], check=True)
    return out


def test_matches_pytorch_aten_engine():
    exe = _aten_binary()
    rng = np.random.default_rng(11)
    cases = rng.integers(0, 2**32, size=(400, 6), dtype=np.uint64)
    cases[:50, 1:4] = 0           # small counters, as the sampler uses them
    cases[50:60, 3] = np.arange(10) % 4  # every tag
    text = "\n".join(" ".join(str(int(x)) for x in row) for row in cases) + "\n"
    res = subprocess.run([exe], input=text, capture_output=True, text=True, check=True)
    ref = np.array([[int(t) for t in line.split()] for line in res.stdout.splitlines()],
                   dtype=np.uint64)
    mine = np.stack(philox.philox4x32_10(*cases.T), axis=1)
    np.testing.assert_array_equal(mine, ref)


def test_uniform_endpoints_and_grid():
    u = philox.uniform_open01(np.array([0, 511, 512, 2**32 - 1], dtype=np.uint64))
    assert u[0] == 2.0 ** -24 and u[1] == 2.0 ** -24
    assert u[2] == 3 * 2.0 ** -24
    assert u[3] == 1.0 - 2.0 ** -24
    assert np.all((u > 0) & (u < 1))
    # every value is exactly representable in fp32
    assert np.all(u.astype(np.float32).astype(np.float64) == u)


def test_uniform_chi_square():
    w = philox.philox4x32_10(np.arange(40000), 3, 7, philox.TAG_BLOCK, 123, 456)
    u = philox.uniform_open01(np.concatenate(w))
    counts, _ = np.histogram(u, bins=64, range=(0.0, 1.0))
    assert scipy.stats.chisquare(counts).pvalue > 1e-4


def test_gumbel_moments():
    w = philox.philox4x32_10(np.arange(50000), 1, 2, philox.TAG_ELEM, 9, 9)
    g = philox.gumbel(np.concatenate(w))
    # standard Gumbel: mean = Euler-Mascheroni, variance = pi^2/6
    assert abs(g.mean() - np.euler_gamma) < 0.02
    assert abs(g.var() - np.pi ** 2 / 6) < 0.05
    assert scipy.stats.kstest(g, "gumbel_r").pvalue > 1e-4
