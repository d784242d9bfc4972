"""GPU parity of the self-conditioning matmul (dg_self_condition) against the
oracle (oracle/selfcond.py).

Tolerance (derived from the arithmetic; the pages fix none): each term
e_v * E[v, n] is formed from e_v = 2^(z c - zmax c) in fp32; rounding the
exponent argument (|t| <= about 40 on these inputs) costs at most 40 * 2^-24,
about 2.4e-6 of the term, after a common factor that the normaliser cancels.
Both factors are split exactly into three bf16 parts and the three cross
products below 2^-16 of the leading one are dropped: at most 3 * 2^-24 of the
term. Sums run in fp32 along chains of at most n = 8192 matrix-core updates
per accumulator plus one addition per vocabulary slice (n <= 8200 for every
launch shape at V <= 262144), so the numerator and the normaliser are each
within (n * 2^-24 + 2.6e-6) of the sum of their terms' magnitudes, and the
ratio within twice that: |gpu - oracle| <= 1.0e-3 * sum_v p_v |E[v, n]|.
That is the worst case; the observed maximum is printed and, being a sum of
independent roundings, sits orders of magnitude below it (checked at 2e-5).
"""
import numpy as np
import pytest
import torch

from canvas_sampler_amd import binding as B
from canvas_sampler_amd import synth
from oracle import selfcond as SC

from gpu_util import gpu, host_values, require_gpu, seeds_tensor

pytestmark = gpu

TOL_BOUND = 1.0e-3
TOL_TYPICAL = 2.0e-5


def _run(L, V, Bn, dtype, d, temps, gen=31, m_max=8.0, rows_check=None, stride=None, pad=3.0):
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V), max_batch=Bn)
    z = torch.cat([synth.margin_logits(gen + c, L, V, m_max=m_max, dtype=dtype, device="cuda")
                   for c in range(Bn)])
    if stride is None and V % 8:
        stride = (V + 7) // 8 * 8   # rows must start on 16-byte boundaries
    if stride is not None:
        buf = torch.full((z.shape[0], stride), pad, dtype=dtype, device="cuda")
        buf[:, :V] = z
        z_in = buf
    else:
        z_in = z
    E = synth.selfcond_embedding(5, V, d, device="cuda")
    rows = Bn * L
    t = torch.tensor(temps, dtype=torch.float32, device="cuda")
    h = torch.empty(rows, device="cuda")
    am = torch.empty(rows, dtype=torch.int32, device="cuda")
    smp = torch.empty(rows, dtype=torch.int32, device="cuda")
    ctx.dg_canvas_stats(z_in, t, 0, seeds_tensor(list(range(Bn))), h, am, smp, batch=Bn)
    out = torch.full((rows, d), float("nan"), device="cuda")
    ctx.dg_self_condition(z_in, t, am, E, out, batch=Bn)
    torch.cuda.synchronize()
    g = out.cpu().numpy().astype(np.float64)
    Eh = E.cpu().numpy().astype(np.float64)
    sel = np.arange(rows) if rows_check is None else np.asarray(sorted(rows_check))
    worst = 0.0
    for i in range(0, len(sel), 64):
        rr = sel[i:i + 64]
        zh = host_values(z[torch.as_tensor(rr, device="cuda")])
        for c in np.unique(rr // L):
            m = (rr // L) == c
            T = np.float32(temps[c])
            want = SC.self_condition(zh[m], T, Eh)
            mag = SC.magnitude(zh[m], T, Eh)
            ratio = np.abs(g[rr[m]] - want) / mag
            assert np.all(np.isfinite(g[rr[m]]))
            assert np.all(ratio <= TOL_BOUND), f"rows {rr[m][np.any(ratio > TOL_BOUND, axis=1)]}"
            worst = max(worst, float(ratio.max()))
    assert worst <= TOL_TYPICAL, worst
    print(f"L={L} V={V} B={Bn} {dtype} d={d}: max |err| / sum p|E| = {worst:.2e} over {len(sel)} rows")
    return g


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V", [2, 100, 1001, 4096, 4100, 70001])
def test_small_and_ragged_vocabularies(V, dtype):
    # ragged V: the last 16-byte piece of a row straddles V (padding follows)
    _run(256, V, 1, dtype, 30, [0.8])


@pytest.mark.parametrize("d", [1, 7, 30, 31])
def test_widths(d):
    _run(100, 4096, 3, torch.bfloat16, d, [0.8, 0.4, 1.7])


def test_full_vocabulary_single_canvas_bf16():
    # the sampling stage of the benchmark step: 256 x 262144 bf16, d = 30
    _run(256, 262144, 1, torch.bfloat16, 30, [0.8], m_max=6.0)


def test_full_vocabulary_batch_fp32_sampled_rows():
    rows = {0, 1, 255, 256, 511, 700, 1023}
    _run(256, 262144, 4, torch.float32, 30, [0.8, 0.6, 0.5, 0.4], rows_check=rows)


def test_one_slice_per_tile_batch():
    # 260 canvases of 256 rows: the row tiles alone fill the grid, so each
    # workgroup covers the whole vocabulary and divides by its own normaliser
    n = 260 * 256
    rows = set(range(0, n, 1021)) | {n - 1}
    _run(256, 4096, 260, torch.bfloat16, 30, [0.4 + 0.4 * (c % 5) / 4 for c in range(260)],
         rows_check=rows)


def test_row_stride_padding_is_ignored():
    _run(64, 1000, 2, torch.bfloat16, 30, [0.8, 0.5], stride=1024)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("pad", [float("nan"), float("inf"), 1.0e30])
def test_row_padding_values_never_count(pad, dtype):
    # whatever the ids between V and the row stride hold (NaN, +inf, a value
    # far above every logit), they take no part in the softmax: V = 1000 with
    # a stride of 1024 puts 24 padding ids in the last 64-id chunk of each row
    _run(64, 1000, 2, dtype, 30, [0.8, 0.5], stride=1024, pad=pad)


def test_rejects_bad_arguments():
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=8, vocab=64), max_batch=1)
    z = torch.zeros(8, 64, device="cuda")
    t = torch.ones(1, device="cuda")
    am = torch.zeros(8, dtype=torch.int32, device="cuda")
    for d in (0, 32):
        E = torch.zeros(64, max(d, 1), device="cuda")
        out = torch.zeros(8, max(d, 1), device="cuda")
        st = B.lib().dg_self_condition(ctx.handle, 1, z.data_ptr(), B.DG_DTYPE_F32, 64, t.data_ptr(),
                                       am.data_ptr(), E.data_ptr(), d, out.data_ptr(), None)
        assert st == B.DG_ERR_INVALID_ARG and "d = " in B.lib().dg_last_error(ctx.handle).decode()
    E = torch.zeros(64, 4, device="cuda")
    out = torch.zeros(8, 4, device="cuda")
    with pytest.raises(B.DgError, match="argmax"):
        ctx._chk(B.lib().dg_self_condition(ctx.handle, 1, z.data_ptr(), B.DG_DTYPE_F32, 64, t.data_ptr(),
                                           None, E.data_ptr(), 4, out.data_ptr(), None))
    # a wave reads 32 rows through one 32-bit buffer range: row_stride * 4
    # bytes must stay below 2^27 (checked before anything is read)
    st = B.lib().dg_self_condition(ctx.handle, 1, z.data_ptr(), B.DG_DTYPE_F32, 1 << 25, t.data_ptr(),
                                   am.data_ptr(), E.data_ptr(), 4, out.data_ptr(), None)
    assert st == B.DG_ERR_UNSUPPORTED and "row_stride" in B.lib().dg_last_error(ctx.handle).decode()


def test_extreme_rows():
    # rows with -inf logits, a near one-hot row (margin 1000), a constant row,
    # and a very low temperature: the softmax stays exact relative to the
    # row's maximum, so every row still matches the oracle
    L, V, d = 64, 4096, 30
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V), max_batch=2)
    z = synth.margin_logits(77, 2 * L, V, m_max=8.0, dtype=torch.float32, device="cuda")
    z[0, ::3] = float("-inf")
    z[1, :V - 1] = float("-inf")          # one finite logit: p is one-hot
    z[2, 17] += 1000.0                     # near one-hot
    z[3, :] = 0.25                         # uniform row
    z[4, 4000:] = float("-inf")            # the tail of the row impossible
    t = torch.tensor([0.8, 0.05], device="cuda")   # canvas 1 at a very low temperature
    E = synth.selfcond_embedding(9, V, d, device="cuda")
    h = torch.empty(2 * L, device="cuda")
    am = torch.empty(2 * L, dtype=torch.int32, device="cuda")
    smp = torch.empty(2 * L, dtype=torch.int32, device="cuda")
    ctx.dg_canvas_stats(z, t, 0, seeds_tensor([1, 2]), h, am, smp, batch=2)
    out = torch.empty(2 * L, d, device="cuda")
    ctx.dg_self_condition(z, t, am, E, out, batch=2)
    torch.cuda.synchronize()
    g = out.cpu().numpy().astype(np.float64)
    zh = host_values(z)
    Eh = E.cpu().numpy().astype(np.float64)
    worst = 0.0
    for c in range(2):
        rows = slice(c * L, (c + 1) * L)
        T = np.float32(t[c].item())
        want = SC.self_condition(zh[rows], T, Eh)
        mag = SC.magnitude(zh[rows], T, Eh)
        assert np.all(np.isfinite(g[rows]))
        ratio = np.abs(g[rows] - want) / mag
        assert np.all(ratio <= TOL_BOUND)
        worst = max(worst, float(ratio.max()))
    assert worst <= TOL_TYPICAL, worst
    assert np.allclose(g[1], Eh[V - 1], rtol=0, atol=1e-6)   # one-hot row picks its embedding row
    print(f"extreme rows: max |err| / sum p|E| = {worst:.2e}")


@pytest.mark.parametrize("Bn,V", [(3, 4096), (520, 1024)])
def test_step_with_selfcond_matches_separate_calls_and_skips_inactive(Bn, V):
    # dg_sampler_step_selfcond = statistics, self-conditioning on their
    # argmax, acceptance: the step outputs equal dg_sampler_step's bit for bit;
    # rows of inactive canvases keep their previous self-conditioning values;
    # active rows match the oracle. B = 520 fills the grid with row tiles, so
    # each workgroup divides in place (no partial tiles).
    L, d = 256, 30
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V), max_batch=Bn)
    z = torch.cat([synth.margin_logits(300 + c, L, V, m_max=8.0, dtype=torch.bfloat16, device="cuda")
                   for c in range(Bn)])
    E = synth.selfcond_embedding(11, V, d, device="cuda")
    t = torch.tensor([0.8 - 0.3 * (c % 3) / 2 for c in range(Bn)], device="cuda")
    seeds = seeds_tensor(list(range(Bn)))
    active = torch.tensor([0 if c % 3 == 1 else 1 for c in range(Bn)], dtype=torch.uint8, device="cuda")
    prev = torch.zeros(Bn * L, dtype=torch.int32, device="cuda")

    def outs():
        return dict(canvas_out=torch.full((Bn * L,), -1, dtype=torch.int32, device="cuda"),
                    argmax_out=torch.full((Bn * L,), -1, dtype=torch.int32, device="cuda"),
                    sample_out=torch.full((Bn * L,), -1, dtype=torch.int32, device="cuda"),
                    entropy_out=torch.full((Bn * L,), -1.0, device="cuda"),
                    accept_out=torch.full((Bn * L,), 9, dtype=torch.uint8, device="cuda"),
                    n_accept_out=torch.full((Bn,), -1, dtype=torch.int32, device="cuda"),
                    stop_out=torch.full((Bn,), 9, dtype=torch.uint8, device="cuda"))

    a, b = outs(), outs()
    ctx.dg_sampler_step(z, t, 2, seeds, ctx.step_out(**a), prev_argmax=prev, active=active)
    sc = torch.full((Bn * L, d), 7.0, device="cuda")
    ctx.dg_sampler_step_selfcond(z, t, 2, seeds, E, sc, ctx.step_out(**b), prev_argmax=prev, active=active)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    g = sc.cpu().numpy().astype(np.float64)
    act = active.cpu().numpy()
    for c in range(Bn):
        rows = slice(c * L, (c + 1) * L)
        if not act[c]:
            assert np.all(g[rows] == 7.0), f"inactive canvas {c} was written"
    check = [c for c in range(Bn) if act[c]][:4]
    Eh = E.cpu().numpy().astype(np.float64)
    worst = 0.0
    for c in check:
        rows = slice(c * L, (c + 1) * L)
        zh = host_values(z[rows])
        T = np.float32(t[c].item())
        ratio = np.abs(g[rows] - SC.self_condition(zh, T, Eh)) / SC.magnitude(zh, T, Eh)
        worst = max(worst, float(ratio.max()))
    assert worst <= TOL_TYPICAL, worst
    print(f"B={Bn} V={V}: step outputs identical; active rows max |err| / sum p|E| = {worst:.2e}")


@pytest.mark.parametrize("offset", [1, 3])
def test_step_with_selfcond_reads_flags_at_any_byte_offset(offset):
    # the canvas flags start `offset` bytes into an allocation: the kernels
    # read each flag through the aligned 32-bit word that holds it, so every
    # canvas must still see its own flag
    L, V, Bn, d = 256, 4096, 6, 30
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V), max_batch=Bn)
    z = torch.cat([synth.margin_logits(500 + c, L, V, m_max=8.0, dtype=torch.bfloat16, device="cuda")
                   for c in range(Bn)])
    E = synth.selfcond_embedding(13, V, d, device="cuda")
    t = torch.tensor([0.8, 0.6, 0.5, 0.7, 0.4, 0.9], device="cuda")
    seeds = seeds_tensor(list(range(Bn)))
    flags = [1, 0, 1, 1, 0, 1]
    buf = torch.full((Bn + 8,), 0xAB, dtype=torch.uint8, device="cuda")
    buf[offset:offset + Bn] = torch.tensor(flags, dtype=torch.uint8, device="cuda")
    active = buf[offset:offset + Bn]
    assert active.data_ptr() % 4 == offset % 4
    prev = torch.zeros(Bn * L, dtype=torch.int32, device="cuda")

    def outs():
        return dict(canvas_out=torch.full((Bn * L,), -1, dtype=torch.int32, device="cuda"),
                    argmax_out=torch.full((Bn * L,), -1, dtype=torch.int32, device="cuda"),
                    sample_out=torch.full((Bn * L,), -1, dtype=torch.int32, device="cuda"),
                    entropy_out=torch.full((Bn * L,), -1.0, device="cuda"),
                    accept_out=torch.full((Bn * L,), 9, dtype=torch.uint8, device="cuda"),
                    n_accept_out=torch.full((Bn,), -1, dtype=torch.int32, device="cuda"),
                    stop_out=torch.full((Bn,), 9, dtype=torch.uint8, device="cuda"))

    a, b = outs(), outs()
    ctx.dg_sampler_step(z, t, 1, seeds, ctx.step_out(**a), prev_argmax=prev, active=active)
    sc = torch.full((Bn * L, d), 7.0, device="cuda")
    ctx.dg_sampler_step_selfcond(z, t, 1, seeds, E, sc, ctx.step_out(**b), prev_argmax=prev, active=active)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k
    g = sc.cpu().numpy().astype(np.float64)
    Eh = E.cpu().numpy().astype(np.float64)
    worst = 0.0
    for c in range(Bn):
        rows = slice(c * L, (c + 1) * L)
        if not flags[c]:
            assert np.all(g[rows] == 7.0), f"inactive canvas {c} was written"
            continue
        zh = host_values(z[rows])
        T = np.float32(t[c].item())
        ratio = np.abs(g[rows] - SC.self_condition(zh, T, Eh)) / SC.magnitude(zh, T, Eh)
        worst = max(worst, float(ratio.max()))
    assert worst <= TOL_TYPICAL, worst
    print(f"flags at byte offset {offset}: step outputs identical; active rows max |err| / sum p|E| = {worst:.2e}")


def test_step_with_selfcond_graph_replays():
    # the step with the matmul (statistics, matmul and its reduction,
    # acceptance) captured into one graph: every replay (new logits copied
    # in, other work and a synchronisation between replays) must equal the
    # eager call bit for bit
    L, V, Bn, d = 256, 4096, 2, 30
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V), max_batch=Bn)
    zs = [torch.cat([synth.margin_logits(700 + 10 * k + c, L, V, m_max=8.0, dtype=torch.bfloat16,
                                         device="cuda") for c in range(Bn)]) for k in range(2)]
    E = synth.selfcond_embedding(17, V, d, device="cuda")
    t = torch.tensor([0.8, 0.5], device="cuda")
    seeds = seeds_tensor([3, 4])
    prev = torch.zeros(Bn * L, dtype=torch.int32, device="cuda")

    def outs():
        return dict(canvas_out=torch.full((Bn * L,), -1, dtype=torch.int32, device="cuda"),
                    argmax_out=torch.full((Bn * L,), -1, dtype=torch.int32, device="cuda"),
                    sample_out=torch.full((Bn * L,), -1, dtype=torch.int32, device="cuda"),
                    entropy_out=torch.full((Bn * L,), -1.0, device="cuda"),
                    accept_out=torch.full((Bn * L,), 9, dtype=torch.uint8, device="cuda"),
                    n_accept_out=torch.full((Bn,), -1, dtype=torch.int32, device="cuda"),
                    stop_out=torch.full((Bn,), 9, dtype=torch.uint8, device="cuda"))

    eager = []
    for k in range(2):
        o = outs()
        sc = torch.full((Bn * L, d), 7.0, device="cuda")
        ctx.dg_sampler_step_selfcond(zs[k], t, 1, seeds, E, sc, ctx.step_out(**o), prev_argmax=prev)
        torch.cuda.synchronize()
        eager.append((o, sc))
    z = zs[0].clone()
    o = outs()
    sc = torch.full((Bn * L, d), 7.0, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ctx.dg_sampler_step_selfcond(z, t, 1, seeds, E, sc, ctx.step_out(**o), prev_argmax=prev)
    torch.cuda.synchronize()
    for k in (0, 1, 0, 1):
        z.copy_(zs[k])
        for v in o.values():
            v.fill_(-1 if v.dtype != torch.uint8 else 9)
        sc.fill_(7.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eo, esc = eager[k]
        for key in o:
            assert torch.equal(o[key], eo[key]), (k, key)
        assert torch.equal(sc, esc), k
    print("graph replays of the step with the matmul equal the eager calls")
