"""GPU parity of the HIP path (through the C ABI) against the oracle."""
import math

import numpy as np
import pytest
import torch

from canvas_sampler_amd import binding as B
from canvas_sampler_amd import synth
from oracle import philox as OP
from oracle import sampler as O

from gpu_util import (accept_tie_clause, check_decision_rules, compare_stats, gpu, host_values, require_gpu,
                      seeds_tensor)

pytestmark = gpu


def _ctx(L, V, max_batch=1, **kw):
    require_gpu()
    return B.Context(B.params_default(canvas_len=L, vocab=V, **kw), max_batch=max_batch)


def _stats(ctx, logits, temps, seeds, step, batch, nsplit=None):
    rows = batch * ctx.L
    h = torch.full((rows,), -1.0, device="cuda")
    am = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    smp = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    if nsplit is not None:
        ctx.set_stats_split(nsplit)
    ctx.dg_canvas_stats(logits, torch.tensor(temps, dtype=torch.float32, device="cuda"), step,
                        seeds_tensor(seeds), h, am, smp, batch=batch)
    torch.cuda.synchronize()
    return h.cpu().numpy(), am.cpu().numpy(), smp.cpu().numpy()


def _padded(z, stride):
    """Copy of z [rows, V] inside a [rows, stride] buffer (padding = garbage 7.0)."""
    buf = torch.full((z.shape[0], stride), 7.0, dtype=z.dtype, device=z.device)
    buf[:, :z.shape[1]] = z
    return buf


def test_c1_stats_match_oracle():
    # single canvas, V = 4096, fp32, margin logits (m ~ U[0,12]), T = 0.8, seed 0
    L, V = 256, 4096
    ctx = _ctx(L, V)
    z = synth.margin_logits(1001, L, V, m_max=12.0, dtype=torch.float32, device="cuda")
    h, am, smp = _stats(ctx, z, [0.8], [0], 0, 1)
    rep = compare_stats(host_values(z), np.float32(0.8), 0, np.arange(L), 0, h, am, smp)
    print("C1 stats", rep)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
# V relative to the 4096-id chunks of the sampling blocks (a block's 8
# stripes arrive as two 4-stripe batches): inside the first batch (1000, 4100,
# 33000, 70001), inside the second (3000, 10340, 39864), on the batch border
# (6144); the block holding V is a wave's first, second (39864, 33000) or
# third block (70001, which also splits each row over two workgroups at L=40).
@pytest.mark.parametrize("V", [2, 7, 100, 1000, 3000, 4100, 6144, 10340, 33000, 39864, 70001])
def test_ragged_vocab(dtype, V):
    L = 40
    ctx = _ctx(L, V)
    per16 = 8 if dtype == torch.bfloat16 else 4
    stride = -(-V // per16) * per16
    z = synth.margin_logits(V, L, V, m_max=5.0, dtype=dtype, device="cuda")
    zp = _padded(z, stride)
    h, am, smp = _stats(ctx, zp, [0.7], [V * 31 + 5], 3, 1)
    compare_stats(host_values(z), np.float32(0.7), V * 31 + 5, np.arange(L), 3, h, am, smp)


# The one-row-per-workgroup kernel splits each SIMD pair's chunks p + 4k
# unevenly between its older and younger wave (the younger takes the last
# ~6/16 of k), and each wave draws its block words from two runs (even and
# odd k) that may start mid-group. Chunk counts that leave a pair with one
# or two chunks, a ragged last chunk, and splits of 32 chunks with a short
# last split.
@pytest.mark.parametrize("V,nsplit,dtype", [
    (5 * 4096, 1, torch.bfloat16),         # pairs of 2, 1, 1, 1 chunks
    (14 * 4096 - 9, 1, torch.bfloat16),    # pairs of 4, 4, 3, 3; the last chunk ragged
    (14 * 4096 - 9, 1, torch.float32),
    (33 * 4096, 2, torch.bfloat16),        # splits of 32 and 1 chunks
    (64 * 4096 + 100, 3, torch.bfloat16),  # splits of 32, 32 and 1 (ragged) chunks
])
def test_simd_pair_shares_match_oracle(V, nsplit, dtype):
    L = 16
    ctx = _ctx(L, V)
    per16 = 8 if dtype == torch.bfloat16 else 4
    stride = -(-V // per16) * per16
    z = synth.margin_logits(V + 17, L, V, m_max=3.0, dtype=dtype, device="cuda")
    zp = _padded(z, stride)
    h, am, smp = _stats(ctx, zp, [0.9], [V * 7 + 1], 5, 1, nsplit=nsplit)
    compare_stats(host_values(z), np.float32(0.9), V * 7 + 1, np.arange(L), 5, h, am, smp)


# Shapes that take the persistent row loop (more rows than compute units, V a
# multiple of 4096, no active mask): each workgroup handles rows b, b + grid,
# ..., and the register ring runs on into the next row. Every row is compared.
@pytest.mark.parametrize("dtype,L,Bn,V", [
    (torch.bfloat16, 256, 4, 262144),  # four rows per workgroup
    (torch.float32, 150, 2, 12288),    # three chunks per row (waves 3-7 idle); rows not a multiple of the grid
    (torch.bfloat16, 100, 3, 4096),    # one chunk per row: the ring slot alternates from row to row
])
def test_row_loop_matches_oracle(dtype, L, Bn, V):
    ctx = _ctx(L, V, max_batch=Bn)
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    rows = Bn * L
    assert rows > cu
    zs = [synth.margin_logits(900 + c, L, V, m_max=4.0, dtype=dtype, device="cuda") for c in range(Bn)]
    z = torch.cat(zs)
    temps = [0.8, 0.5, 1.3, 0.7][:Bn]
    seeds = [11, 2**40 + 3, 7, 99][:Bn]
    h, am, smp = _stats(ctx, z, temps, seeds, 4, Bn)
    # every row: workgroup borders, loop-iteration borders and the rest
    res = _oracle_rows(z, temps, seeds, 4, L)
    for c in range(Bn):
        sl = slice(c * L, (c + 1) * L)
        _check_rows(res[c], h[sl], am[sl], smp[sl], f"canvas {c}")


def test_row_stride_padding_is_ignored():
    L, V = 32, 4096
    ctx = _ctx(L, V)
    z = synth.margin_logits(7, L, V, dtype=torch.bfloat16, device="cuda")
    zp = _padded(z, V + 64)
    zp[:, V:] = 1e4   # huge values in the padding must not be read
    h, am, smp = _stats(ctx, zp, [0.8], [1], 0, 1)
    compare_stats(host_values(z), np.float32(0.8), 1, np.arange(L), 0, h, am, smp)


def test_neg_inf_and_degenerate_rows():
    L, V = 8, 70000
    ctx = _ctx(L, V)
    z = torch.randn(L, V, device="cuda")
    z[0, :] = float("-inf")
    z[0, 12345] = 0.5                       # single finite logit
    z[1, :40000] = float("-inf")            # whole chunks of -inf
    z[2, ::3] = float("-inf")               # scattered -inf
    z[3, :] = 1.0                           # constant row: H = ln V, argmax 0
    z[4, :] = -3.0e4
    z[4, 69999] = 0.0                       # finite one-hot at the last id
    z[5, 100:200] = 50.0                    # 100-way tie at the max
    h, am, smp = _stats(ctx, z, [0.8], [99], 2, 1)
    zh = host_values(z)
    compare_stats(zh, np.float32(0.8), 99, np.arange(L), 2, h, am, smp)
    assert smp[0] == 12345 and h[0] == 0.0
    assert am[3] == 0 and abs(h[3] - math.log(V)) < 1e-4
    assert am[4] == 69999 and smp[4] == 69999 and h[4] == 0.0
    assert am[5] == 100 and 100 <= smp[5] < 200 and abs(h[5] - math.log(100)) < 1e-4


def test_batch_of_canvases_with_own_temperatures_and_seeds():
    L, V, Bn = 64, 40000, 3
    ctx = _ctx(L, V, max_batch=4)
    zs = [synth.margin_logits(50 + c, L, V, m_max=3.0, dtype=torch.bfloat16, device="cuda")
          for c in range(Bn)]
    z = torch.cat(zs)
    temps = [0.8, 0.4, 2.0]
    seeds = [5, 2**63 + 12345, 2**64 - 1]
    h, am, smp = _stats(ctx, z, temps, seeds, 7, Bn)
    for c in range(Bn):
        sl = slice(c * L, (c + 1) * L)
        compare_stats(host_values(zs[c]), np.float32(temps[c]), seeds[c], np.arange(L), 7,
                      h[sl], am[sl], smp[sl])


def _oracle_rows(z, temps, seeds, step, L):
    """Oracle row statistics of every row of z ([B*L, V] on the GPU), canvas c
    with temperature temps[c] and seed seeds[c]; all rows, thread pool."""
    from oracle import parallel as OPAR
    n = z.shape[0] // L
    hosts = [z[c * L:(c + 1) * L].to("cpu").to(torch.float32).numpy() for c in range(n)]
    jobs = [dict(rows=lambda r0, r1, zc=hosts[c]: zc[r0:r1], L=L, V=z.shape[1], temp=np.float32(temps[c]),
                 seed=seeds[c], step=step, prev_argmax=None) for c in range(n)]
    return OPAR.steps(jobs)


def _check_rows(o, h, am, smp, label):
    """All rows of one canvas against oracle.parallel's record o: |dH| <= 1e-4,
    argmax exact, every sample difference an oracle near-tie. Returns
    (max |dH|, sample near-tie mismatches)."""
    from gpu_util import H_TOL, near_tie
    dh = float(np.max(np.abs(h.astype(np.float64) - o["entropy"])))
    assert dh <= H_TOL, f"{label}: entropy error {dh:.3g}"
    bad = np.flatnonzero(am != o["argmax"])
    assert bad.size == 0, f"{label}: argmax differs at rows {bad[:10]}"
    ties = near_tie(o["block_best"], o["block_gap"]) | near_tie(o["elem_best"], o["elem_gap"])
    mism = smp != o["sample"]
    hard = np.flatnonzero(mism & ~ties)
    assert hard.size == 0, f"{label}: sample differs at rows {hard[:10]} that are not near-ties"
    return dh, int((mism & ties).sum())


def test_full_vocab_every_split_all_rows():
    # the launch shape of the single-canvas bf16 benchmark (B=1, V=262144) and
    # every split count, all 256 rows against the oracle: argmax equal, the
    # entropy within 1e-4, and every sample that differs from the oracle's (or
    # between split counts) an oracle near-tie
    L, V = 256, 262144
    ctx = _ctx(L, V)
    z = synth.sharpening_logits(1002, 3, L, V, m0_max=6.0, dtype=torch.bfloat16, device="cuda")
    o = _oracle_rows(z, [0.7], [0], 3, L)[0]
    base = None
    for nsplit in (0, 1, 2, 4, 8):
        h, am, smp = _stats(ctx, z, [0.7], [0], 3, 1, nsplit=nsplit)
        dh, ties = _check_rows(o, h, am, smp, f"nsplit {nsplit}")
        print(f"nsplit {nsplit}: max |dH| {dh:.2e}, sample near-tie mismatches {ties}")
        if base is None:
            base = (h, am, smp)
        else:
            assert np.array_equal(am, base[1])
            assert np.max(np.abs(h - base[0])) < 1e-5
    ctx.set_stats_split(0)


def test_init_canvas_matches_oracle():
    L, V = 256, 262144
    ctx = _ctx(L, V, max_batch=3)
    seeds = [0, 1, 2**64 - 2]
    canvas = torch.full((3, L), -1, dtype=torch.int32, device="cuda")
    ctx.dg_canvas_init(seeds_tensor(seeds), canvas)
    torch.cuda.synchronize()
    for c, s in enumerate(seeds):
        assert np.array_equal(canvas[c].cpu().numpy(), O.init_canvas(s, L, V))


def _accept_case(rng, L, kind):
    if kind == "random":
        return rng.exponential(rng.choice([0.005, 0.03, 0.3]), size=L).astype(np.float32)
    if kind == "ties":
        h = np.round(rng.exponential(0.02, size=L), 3).astype(np.float32)
        h[rng.integers(0, L, size=L // 3)] = 0.0
        return h
    if kind == "uniform":
        return np.full(L, np.float32(math.log(262144)))
    if kind == "zeros":
        return np.zeros(L, dtype=np.float32)
    if kind == "equal_small":
        return np.full(L, np.float32(0.03125))
    if kind.startswith("c"):
        # n positions at or below the bound b = 0.1, the rest above it: the
        # acceptance's one-wave path holds up to 63 such positions, the full
        # sort takes over from 64. "cN" spreads the small ones up to b, so the
        # prefix stops inside them; "cN_all" makes them tiny, so the prefix
        # runs through all of them and takes the smallest entropy above b too
        n = min(int(kind[1:].split("_")[0]), L)
        h = (1.0 + rng.random(L)).astype(np.float32)
        small = rng.choice(L, size=n, replace=False)
        h[small] = (rng.random(n) * (1e-5 if kind.endswith("_all") else 0.1)).astype(np.float32)
        return h
    raise ValueError(kind)


@pytest.mark.parametrize("L", [256, 100, 1])
def test_accept_renoise_stop_exact_from_given_entropies(L):
    V = 262144
    # c15/c16, c31/c32: the one-wave path's sorting network grows at 16 and
    # 32 keys (the candidates plus the smallest key above b)
    kinds = ["random", "ties", "uniform", "zeros", "equal_small", "random", "c63", "c64", "c65", "c63_all",
             "c64_all", "c1_all", "c1", "c15", "c16", "c31", "c32", "c15_all", "c16_all", "c31_all", "c32_all"]
    Bn = len(kinds)
    ctx = _ctx(L, V, max_batch=Bn)
    rng = np.random.default_rng(L)
    H = np.stack([_accept_case(rng, L, k) for k in kinds])
    am = rng.integers(0, V, size=(Bn, L)).astype(np.int32)
    prev = am.copy()
    prev[1, 0] ^= 1                          # canvas 1 not stable
    smp = rng.integers(0, V, size=(Bn, L)).astype(np.int32)
    seeds = [11, 12, 13, 14, 15, 2**63, 16, 17, 18, 19, 20, 21] + list(range(22, 22 + Bn - 12))
    step = 5
    dev = lambda a, dt: torch.as_tensor(a, dtype=dt, device="cuda")
    canvas = torch.full((Bn, L), -1, dtype=torch.int32, device="cuda")
    acc = torch.full((Bn, L), 7, dtype=torch.uint8, device="cuda")
    nacc = torch.full((Bn,), -1, dtype=torch.int32, device="cuda")
    meanh = torch.full((Bn,), -1.0, device="cuda")
    stop = torch.full((Bn,), 7, dtype=torch.uint8, device="cuda")
    out = ctx.step_out(canvas, accept_out=acc, n_accept_out=nacc, mean_entropy_out=meanh,
                       stop_out=stop)
    ctx.dg_accept_renoise(dev(H.ravel(), torch.float32), dev(am.ravel(), torch.int32),
                          dev(smp.ravel(), torch.int32), step, seeds_tensor(seeds), out,
                          prev_argmax=dev(prev.ravel(), torch.int32))
    torch.cuda.synchronize()
    for c in range(Bn):
        mask, k = O.accept(H[c].astype(np.float64), np.float32(0.1))
        ren = O.uniform_tokens(seeds[c], L, step, V, OP.TAG_RENOISE)
        want = np.where(mask, smp[c], ren)
        assert nacc[c].item() == k
        assert np.array_equal(acc[c].cpu().numpy().astype(bool), mask)
        assert np.array_equal(canvas[c].cpu().numpy(), want)
        mh = float(np.mean(H[c].astype(np.float64)))
        assert abs(meanh[c].item() - mh) < 1e-6 * max(1.0, mh)
        want_stop = O.stop_test(am[c], prev[c], mh, np.float32(0.005))
        assert bool(stop[c].item()) == want_stop
    assert stop[3].item() == 1 and stop[1].item() == 0   # zeros canvas stops, canvas 1 changed


def test_inactive_canvases_are_untouched():
    L, V = 64, 4096
    ctx = _ctx(L, V, max_batch=2)
    z = synth.margin_logits(3, 2 * L, V, device="cuda")
    temps = torch.tensor([0.8, 0.8], device="cuda")
    active = torch.tensor([0, 1], dtype=torch.uint8, device="cuda")
    canvas = torch.full((2, L), -5, dtype=torch.int32, device="cuda")
    am = torch.full((2 * L,), -5, dtype=torch.int32, device="cuda")
    stop = torch.full((2,), 9, dtype=torch.uint8, device="cuda")
    out = ctx.step_out(canvas, argmax_out=am, stop_out=stop)
    ctx.dg_sampler_step(z, temps, 0, seeds_tensor([1, 2]), out, active=active)
    torch.cuda.synchronize()
    assert torch.all(canvas[0] == -5) and torch.all(am[:L] == -5) and stop[0].item() == 9
    assert torch.all(canvas[1] >= 0) and torch.all(am[L:] >= 0) and stop[1].item() == 0


def test_sampler_step_full_outputs_match_oracle_c1():
    L, V = 256, 4096
    ctx = _ctx(L, V)
    z = synth.margin_logits(1001, L, V, m_max=12.0, dtype=torch.float32, device="cuda")
    t = torch.tensor([0.8], device="cuda")
    bufs = dict(canvas_out=torch.empty(L, dtype=torch.int32, device="cuda"),
                argmax_out=torch.empty(L, dtype=torch.int32, device="cuda"),
                sample_out=torch.empty(L, dtype=torch.int32, device="cuda"),
                accept_out=torch.empty(L, dtype=torch.uint8, device="cuda"),
                entropy_out=torch.empty(L, device="cuda"),
                n_accept_out=torch.empty(1, dtype=torch.int32, device="cuda"),
                mean_entropy_out=torch.empty(1, device="cuda"),
                stop_out=torch.empty(1, dtype=torch.uint8, device="cuda"))
    ctx.dg_sampler_step(z, t, 0, seeds_tensor([0]), ctx.step_out(**bufs))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in bufs.items()}
    ref = O.step(host_values(z), np.float32(0.8), 0, 0)
    compare_stats(host_values(z), np.float32(0.8), 0, np.arange(L), 0, g["entropy_out"],
                  g["argmax_out"], g["sample_out"])
    dh = float(np.max(np.abs(g["entropy_out"] - ref["entropy"])))
    if not np.array_equal(g["accept_out"].astype(bool), ref["accept"]) or g["n_accept_out"][0] != ref["n_accept"]:
        clause = accept_tie_clause(ref["entropy"], float(np.float32(0.1)), dh)
        assert clause, f"acceptance differs from the oracle's without a near-tie (max |dH| {dh:.3g})"
        print("C1 acceptance near-tie:", clause)
    # the GPU's decisions obey the rules given its own statistics
    ren = O.uniform_tokens(0, L, 0, V, OP.TAG_RENOISE)
    k = check_decision_rules(g["entropy_out"], g["accept_out"], g["n_accept_out"][0], g["sample_out"],
                             g["canvas_out"], ren, g["mean_entropy_out"][0], g["stop_out"][0], None,
                             g["argmax_out"], float(np.float32(0.1)), float(np.float32(0.005)))
    assert g["stop_out"][0] == 0
    print("C1 step: n_accept", k, "max dH", dh)


def test_split_rows_repeatable_over_many_launches():
    # rows split over several workgroups are finished by the last of them,
    # which reads the others' partials after a release/acquire hand-off; a
    # missing ordering would show up as a run whose integers or entropies
    # differ from the others. 600 launches, bit for bit.
    L, V = 256, 262144
    ctx = _ctx(L, V)
    zs = [synth.sharpening_logits(1002, s, L, V, m0_max=6.0, dtype=torch.bfloat16, device="cuda")
          for s in (0, 5)]
    t = torch.tensor([0.7], device="cuda")
    seeds = seeds_tensor([3])
    n = 300
    for nsplit in (2, 4):
        ctx.set_stats_split(nsplit)
        h = torch.empty(n, L, device="cuda")
        am = torch.empty(n, L, dtype=torch.int32, device="cuda")
        smp = torch.empty(n, L, dtype=torch.int32, device="cuda")
        for i in range(n):
            ctx.dg_canvas_stats(zs[i & 1], t, 1, seeds, h[i], am[i], smp[i])
        torch.cuda.synchronize()
        for par in (0, 1):
            idx = torch.arange(par, n, 2, device="cuda")
            for x in (h, am, smp):
                sel = x[idx]
                assert torch.equal(sel, sel[:1].expand_as(sel)), f"nsplit {nsplit}: launches differ"
    ctx.set_stats_split(0)


def test_c3_sixteen_canvases_step_matches_oracle():
    # C3 at its full size (16 canvases x 256 positions x 262144 bf16, the
    # sharpening stand-in with m0 ~ U[0, 8] and per-canvas generator seeds,
    # sampler seeds c): one whole step through the persistent row loop (no
    # active mask), the launch the benchmark's B = 16 line times. All 4096
    # rows against the oracle; each canvas's commits, new canvas and stop
    # against the oracle's (near-ties counted) and against the rules.
    from full_parity import Tally, compare_step
    L, V, Bn = 256, 262144, 16
    ctx = _ctx(L, V, max_batch=Bn)
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert Bn * L > cu
    step = 6  # margins m0 + 9: a mix of confident and open positions
    z = torch.cat([synth.sharpening_logits((1003 << 32) | c, step, L, V, m0_max=8.0, dtype=torch.bfloat16,
                                           device="cuda") for c in range(Bn)])
    t = B.dg_temperature(B.params_default(canvas_len=L, vocab=V, temp_steps=16), step)
    temps = torch.full((Bn,), t, device="cuda")
    seeds = list(range(Bn))
    bufs = dict(canvas_out=torch.empty(Bn * L, dtype=torch.int32, device="cuda"),
                argmax_out=torch.empty(Bn * L, dtype=torch.int32, device="cuda"),
                sample_out=torch.empty(Bn * L, dtype=torch.int32, device="cuda"),
                accept_out=torch.empty(Bn * L, dtype=torch.uint8, device="cuda"),
                entropy_out=torch.empty(Bn * L, device="cuda"),
                n_accept_out=torch.empty(Bn, dtype=torch.int32, device="cuda"),
                mean_entropy_out=torch.empty(Bn, device="cuda"),
                stop_out=torch.empty(Bn, dtype=torch.uint8, device="cuda"))
    ctx.dg_sampler_step(z, temps, step, seeds_tensor(seeds), ctx.step_out(**bufs))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in bufs.items()}
    res = _oracle_rows(z, [t] * Bn, seeds, step, L)
    tally = Tally("C3 one step, row loop")
    for c in range(Bn):
        sl = slice(c * L, (c + 1) * L)
        gc = dict(entropy=g["entropy_out"][sl], argmax=g["argmax_out"][sl], sample=g["sample_out"][sl],
                  accept=g["accept_out"][sl], n_accept=g["n_accept_out"][c], canvas=g["canvas_out"][sl],
                  mean_entropy=g["mean_entropy_out"][c], stop=g["stop_out"][c])
        compare_step(gc, res[c], f"C3 canvas {c} step {step}", tally, np.float32(0.1), np.float32(0.005))
        check_decision_rules(g["entropy_out"][sl], g["accept_out"][sl].astype(bool), g["n_accept_out"][c],
                             g["sample_out"][sl], g["canvas_out"][sl], res[c]["renoise"], g["mean_entropy_out"][c],
                             g["stop_out"][c], None, g["argmax_out"][sl], float(np.float32(0.1)),
                             float(np.float32(0.005)))
    print("C3 step: 16 canvases, commits", g["n_accept_out"].tolist())
    tally.report()
