"""Pins of the oracle's per-position statistics, sampling protocol, acceptance,
renoise, stop test and schedule against closed forms, library routines other
than the ones the oracle calls, brute force and distribution tests."""
import itertools
import math

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import philox
from oracle import sampler as O


# ---------------------------------------------------------------- schedule --
def test_schedule_matches_linspace():
    for n in (48, 16, 2):
        ref = np.linspace(np.float64(np.float32(0.8)), np.float64(np.float32(0.4)), n)
        got = np.array([O.temperature(s, 0.8, 0.4, n) for s in range(n)], dtype=np.float32)
        ulp = np.spacing(ref.astype(np.float32))
        assert np.all(np.abs(got.astype(np.float64) - ref) <= ulp)
        assert got[0] == np.float32(0.8) and got[-1] == np.float32(0.4)
        assert np.all(np.diff(got) < 0)


def test_schedule_clamps_and_single_step():
    assert O.temperature(100, 0.8, 0.4, 16) == np.float32(0.4)
    assert O.temperature(0, 0.8, 0.4, 1) == np.float32(0.8)
    assert O.temperature(5, 0.8, 0.4, 1) == np.float32(0.8)


# ----------------------------------------------------------------- entropy --
@pytest.mark.parametrize("vocab", [2, 1000, 4096, 262144])
def test_entropy_constant_logits_is_ln_v(vocab):
    z = np.full((3, vocab), 1.25)
    h = O.entropy(z, np.float32(0.8))
    np.testing.assert_allclose(h, math.log(vocab), rtol=0, atol=1e-12)


def test_entropy_uniform_691_nats_at_v1000():
    # "DiffusionGemma Lab" EXP A: an untrained model's mean entropy sits at the
    # uniform value, printed as 6.91 nats (ln 1000 = 6.9078).
    h = O.entropy(np.zeros((1, 1000)), np.float32(0.8))[0]
    assert round(h, 2) == 6.91


def test_entropy_one_hot_and_k_way_ties():
    z = np.full((4, 700), -np.inf)
    z[0, 17] = 3.0                        # one-hot, other ids impossible
    z[1, [5, 300, 699]] = 2.0             # 3 equal maxima
    z[2, :] = -3.0e4
    z[2, 400] = 0.0                       # finite one-hot: the rest underflows
    z[3, :8] = 0.5                        # 8 equal maxima
    h = O.entropy(z, np.float32(0.8))
    np.testing.assert_allclose(h, [0.0, math.log(3), 0.0, math.log(8)], atol=1e-12)
    assert np.all(np.signbit(h) == False)  # noqa: E712  (+0, never -0)


def test_entropy_matches_scipy_on_random_rows():
    rng = np.random.default_rng(0)
    z = rng.normal(size=(20, 3000)) * rng.uniform(0.1, 5, size=(20, 1))
    for t in (np.float32(0.8), np.float32(0.4), np.float32(1.7)):
        p = scipy.special.softmax(z / np.float64(t), axis=1)
        ref = scipy.stats.entropy(p, axis=1)
        np.testing.assert_allclose(O.entropy(z, t), ref, rtol=1e-11, atol=1e-12)


def test_entropy_uses_temperature():
    z = np.random.default_rng(1).normal(size=(1, 500))
    assert O.entropy(z, np.float32(0.4))[0] < O.entropy(z, np.float32(0.8))[0]


# ------------------------------------------------------------------ argmax --
def test_argmax_lowest_index_on_ties_brute_force():
    rng = np.random.default_rng(2)
    z = rng.integers(-3, 3, size=(200, 37)).astype(np.float64)
    got = O.argmax_raw(z)
    for r in range(z.shape[0]):
        best = 0
        for v in range(1, z.shape[1]):
            if z[r, v] > z[r, best]:
                best = v
        assert got[r] == best


def test_argmax_planted():
    z = np.zeros((3, 262144), dtype=np.float32)
    z[0, 262143] = 1.0
    z[1, [9, 100000]] = 2.0
    z[2, :] = -1.0
    z[2, 0] = -0.5
    assert list(O.argmax_raw(z)) == [262143, 9, 0]


# ------------------------------------------------------ block geometry ------
@pytest.mark.parametrize("vocab", [1, 7, 100, 512, 4096, 5000, 32768, 40000])
def test_blocks_partition_the_vocabulary(vocab):
    n_chunk = -(-vocab // 4096)
    seen = np.zeros(vocab, dtype=int)
    for j in range(n_chunk * O.SLOTS):
        mem = O.block_members(j, vocab)
        assert np.all(np.diff(mem) > 0)
        assert len(mem) <= 64
        seen[mem] += 1
        assert np.all(O.block_index(mem) == j)
    assert np.all(seen == 1)


def test_block_index_brute_force():
    # block = (chunk of 4096 ids, position of the 8-id slot in its stripe)
    for v in list(range(0, 5000)) + [8191, 8192, 8199, 32767, 32768, 65535, 262143]:
        chunk = v // 4096
        slot = (v % 512) // 8
        assert O.block_index(v) == 64 * chunk + slot


def test_block_logsumexp_brute_force():
    rng = np.random.default_rng(3)
    vocab = 33000
    x = rng.normal(size=(2, vocab)) * 3
    x[1, 40:80] = -np.inf
    lse = O.block_logsumexp(x)
    assert lse.shape == (2, 9 * 64)
    for r in range(2):
        for j in range(9 * 64):
            mem = O.block_members(j, vocab)
            if len(mem) == 0:
                assert lse[r, j] == -np.inf
            else:
                ref = scipy.special.logsumexp(x[r, mem])
                assert abs(lse[r, j] - ref) < 1e-10
    total = scipy.special.logsumexp(lse, axis=1)
    np.testing.assert_allclose(total, scipy.special.logsumexp(x, axis=1), rtol=1e-12)


# ---------------------------------------------------------------- sampling --
def _designed_row(vocab, ids, vals):
    z = np.full(vocab, -np.inf)
    z[ids] = vals
    return z


@pytest.mark.parametrize("sampler_fn", [O.sample_two_level, O.sample_per_element])
def test_sample_frequencies_match_softmax(sampler_fn):
    # mass on ids in different slots, stripes and chunks
    vocab = 40000
    ids = np.array([3, 9, 700, 701, 4095, 12345, 33000, 39999])
    vals = np.array([0.0, 0.4, -0.3, 1.0, 0.2, -1.0, 0.7, 0.1])
    temp = np.float32(0.8)
    p = scipy.special.softmax(vals / np.float64(temp))
    z = np.tile(_designed_row(vocab, ids, vals), (100, 1))
    draws = []
    for s in range(30):
        draws.append(sampler_fn(z, temp, 77, np.arange(100), s))
    draws = np.concatenate(draws)
    counts = np.array([(draws == i).sum() for i in ids])
    assert counts.sum() == len(draws)
    assert scipy.stats.chisquare(counts, p * len(draws)).pvalue > 1e-4


def test_sample_dense_row_frequencies():
    # every id has mass; V spans several blocks; compare grouped frequencies
    vocab = 1500
    rng = np.random.default_rng(4)
    row = rng.normal(size=vocab) * 0.5
    row[[10, 600, 1400]] += 4.0
    temp = np.float32(0.8)
    p = scipy.special.softmax(row / np.float64(temp))
    z = np.tile(row, (200, 1))
    draws = np.concatenate([O.sample_two_level(z, temp, 5, np.arange(200), s) for s in range(25)])
    edges = [0, 10, 11, 600, 601, 1400, 1401, vocab]
    obs = np.array([((draws >= a) & (draws < b)).sum() for a, b in zip(edges[:-1], edges[1:])])
    exp = np.array([p[a:b].sum() for a, b in zip(edges[:-1], edges[1:])]) * len(draws)
    assert scipy.stats.chisquare(obs, exp).pvalue > 1e-4


@pytest.mark.parametrize("vocab", [8, 100, 4096, 40000, 262144])
def test_sample_planted_dominant_id(vocab):
    rng = np.random.default_rng(vocab)
    targets = sorted(set([0, vocab - 1] + list(rng.integers(0, vocab, size=6))))
    z = np.zeros((len(targets), vocab))
    for r, t in enumerate(targets):
        z[r, t] = 200.0
    got = O.sample_two_level(z, np.float32(0.8), 1, np.arange(len(targets)), 3)
    assert list(got) == targets


def test_sample_single_support():
    z = _designed_row(5000, [4321], [0.0])[None, :]
    for s in range(5):
        assert O.sample_two_level(z, np.float32(0.8), s, [0], s)[0] == 4321


def test_sample_depends_on_seed_position_step():
    z = np.zeros((1, 262144))
    base = O.sample_two_level(z, np.float32(0.8), 1, [0], 0)[0]
    others = [O.sample_two_level(z, np.float32(0.8), 2, [0], 0)[0],
              O.sample_two_level(z, np.float32(0.8), 1, [1], 0)[0],
              O.sample_two_level(z, np.float32(0.8), 1, [0], 1)[0]]
    assert all(o != base for o in others)


# -------------------------------------------------------------- acceptance --
def _brute_force_k(h, bound):
    """Largest |U| over all subsets with sum(U) - max(U) <= bound."""
    best = 0
    L = len(h)
    for k in range(1, L + 1):
        for sub in itertools.combinations(range(L), k):
            vals = h[list(sub)]
            if vals.sum() - vals.max() <= bound:
                best = k
                break
    return best


def test_accept_brute_force_small_canvases():
    rng = np.random.default_rng(6)
    for trial in range(120):
        L = int(rng.integers(1, 11))
        h = rng.exponential(scale=rng.choice([0.01, 0.05, 0.3]), size=L)
        if trial % 4 == 0:
            h[rng.integers(0, L, size=L // 2)] = 0.0      # exact ties at zero
        if trial % 5 == 0:
            h = np.round(h, 2)                            # more ties
        bound = float(np.float32(rng.choice([0.0, 0.05, 0.1, 0.5])))
        mask, k = O.accept(h, bound)
        assert k == _brute_force_k(h, bound)
        assert mask.sum() == k >= 1
        # accepted set = the k lowest (entropy, position) pairs
        order = sorted(range(L), key=lambda i: (h[i], i))
        assert set(np.flatnonzero(mask)) == set(order[:k])


def test_accept_equal_entropies_closed_form():
    # all entropies equal to h: accept min(L, floor(b/h) + 1)
    for h, b, L, want in [(0.03125, 0.1, 256, 4), (0.5, 0.1, 256, 1),
                          (0.0, 0.1, 256, 256), (0.025, 0.1, 3, 3), (0.1, 0.1, 10, 2)]:
        mask, k = O.accept(np.full(L, h), np.float64(b))
        assert k == want
        assert np.all(np.flatnonzero(mask) == np.arange(want))  # ties -> lowest positions


def test_accept_at_least_one_and_monotone_in_bound():
    rng = np.random.default_rng(7)
    h = rng.exponential(0.05, size=256)
    ks = [O.accept(h, b)[1] for b in (0.0, 0.01, 0.1, 1.0, 10.0)]
    assert ks[0] >= 1 and all(a <= b for a, b in zip(ks, ks[1:]))
    assert O.accept(np.full(256, 12.0), 0.1)[1] == 1


# -------------------------------------------------------- renoise and init --
def test_uniform_tokens_chi_square_and_range():
    toks = np.concatenate([O.uniform_tokens(s, 256, 3, 16, philox.TAG_RENOISE) for s in range(200)])
    assert toks.min() >= 0 and toks.max() < 16
    counts = np.bincount(toks, minlength=16)
    assert scipy.stats.chisquare(counts).pvalue > 1e-4


def test_uniform_tokens_top_bits_for_power_of_two_vocab():
    k0, k1 = philox.seed_key(0x1234_5678_9ABC_DEF0)
    w0 = philox.philox4x32_10(0, np.arange(256), 5, philox.TAG_RENOISE, k0, k1)[0]
    got = O.uniform_tokens(0x1234_5678_9ABC_DEF0, 256, 5, 262144, philox.TAG_RENOISE)
    assert np.array_equal(got, (w0 >> np.uint64(14)).astype(np.int64))


def test_init_canvas_in_range_and_seeded():
    a = O.init_canvas(3, 256, 262144)
    assert a.min() >= 0 and a.max() < 262144
    assert np.array_equal(a, O.init_canvas(3, 256, 262144))
    assert not np.array_equal(a, O.init_canvas(4, 256, 262144))


# ---------------------------------------------------------------- stop test --
def test_stop_truth_table():
    a = np.arange(8)
    b = a.copy()
    b[3] = 99
    assert O.stop_test(a, a.copy(), 0.001, 0.005) is True
    assert O.stop_test(a, None, 0.001, 0.005) is False          # no previous step
    assert O.stop_test(a, b, 0.001, 0.005) is False             # argmax changed
    assert O.stop_test(a, a.copy(), 0.01, 0.005) is False       # not confident
    assert O.stop_test(a, a.copy(), float(np.float32(0.005)), np.float32(0.005)) is False  # strict


def test_block_words_are_distinct_draws():
    # four blocks share a Philox call, each taking its own word: no two
    # blocks of a row may end up with the same (counter, word) pair, and the
    # words match the Philox outputs of that counter
    j = np.arange(8192, dtype=np.int64)
    pairs = set(zip((j & ~0x600).tolist(), ((j >> 9) & 3).tolist()))
    assert len(pairs) == len(j)
    w = O.block_word(j, 5, 3, 11, 22)
    for q in range(4):
        sel = j[((j >> 9) & 3) == q]
        ref = philox.philox4x32_10(sel & ~0x600, 5, 3, philox.TAG_BLOCK, 11, 22)[q]
        assert np.array_equal(w[sel], ref)
    # distinct blocks get distinct words (collisions among 8192 32-bit words are unlikely)
    assert len(np.unique(w)) > 8180
