"""GPU parity of the LM-head configuration through the C ABI: the product
(dg_lmhead_logits) against the oracle's exact products, and the fused step
(dg_lmhead_sampler_step, statistics inside the product's epilogue) against the
oracle's sampler on the product's own logits.

Logit tolerance. The GPU sums K bf16 products with fp32 accumulation on the
matrix cores (32 products per instruction, K/32 instructions chained). To
first order in u = 2^-24 the error of such a sum is at most
(K/32 + 31) * u * sum_k |h_k w_k|: at most 31 roundings inside one
instruction's 32-term sum, one per chained accumulation. Every logit is checked
against that bound; the measured maximum is printed (it is far smaller).
"""
import ctypes

import numpy as np
import pytest
import torch

from canvas_sampler_amd import binding as B
from canvas_sampler_amd import synth
from oracle import lmhead as OL
from oracle import sampler as O

from gpu_util import check_decision_rules, compare_stats, gpu, require_gpu, seeds_tensor

pytestmark = gpu

U = 2.0 ** -24


def _bound(h, w, chunk=16384):
    """First-order error bound of fp32 MFMA accumulation, per logit."""
    k = h.shape[1]
    ah = np.abs(h.astype(np.float64))
    out = np.empty((h.shape[0], w.shape[1]))
    for c0 in range(0, w.shape[1], chunk):
        out[:, c0:c0 + chunk] = ah @ np.abs(w[:, c0:c0 + chunk].astype(np.float64))
    return (k / 32 + 31) * U * out


def _f32(t):
    """Exact fp32 host copy of a bf16 tensor."""
    return t.detach().to(torch.float32).cpu().numpy()


def _check_logits(gpu_z, h, w, label, exact=None):
    if exact is None:
        exact = OL.logits(h, w)
    err = np.abs(gpu_z.astype(np.float64) - exact)
    bound = _bound(h, w)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    assert np.all(err <= bound), (f"{label}: logit error {err[worst]:.3g} above bound {bound[worst]:.3g} "
                                  f"at {worst}")
    print(f"{label}: max |dz| {err.max():.3g} (bound >= {bound.min():.3g})")
    return exact, err


@pytest.mark.parametrize("rows,k,vocab", [(1, 64, 8), (300, 128, 1000), (513, 192, 2056),
                                          (256, 2048, 4096)])
def test_lmhead_logits_ragged_shapes(rows, k, vocab):
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=1, vocab=vocab), max_batch=1)
    h, w = synth.lmhead_operands(2000 + rows, rows, k, vocab, device="cuda")
    ld = vocab + 12   # padded rows: the columns past V must stay untouched
    z = torch.full((rows, ld), float("nan"), device="cuda")
    ctx.dg_lmhead_logits(h, w, z)
    torch.cuda.synchronize()
    zh = z.cpu().numpy()
    assert np.all(np.isnan(zh[:, vocab:])), "columns past V were written"
    _check_logits(zh[:, :vocab], _f32(h), _f32(w), f"{rows}x{k}x{vocab}")


def test_lmhead_rejects_unsupported_shapes():
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=4, vocab=1000), max_batch=1)
    h, w = synth.lmhead_operands(1, 4, 96, 1000, device="cuda")
    z = torch.empty(4, 1000, device="cuda")
    with pytest.raises(B.DgError) as e:
        ctx.dg_lmhead_logits(h, w, z)
    assert e.value.status == B.DG_ERR_UNSUPPORTED and "hidden_dim" in str(e.value)
    ctx2 = B.Context(B.params_default(canvas_len=4, vocab=1001), max_batch=1)
    h2, w2 = synth.lmhead_operands(1, 4, 64, 1001, device="cuda")
    with pytest.raises(B.DgError) as e:
        ctx2.dg_lmhead_logits(h2, w2, torch.empty(4, 1004, device="cuda"))
    assert e.value.status == B.DG_ERR_UNSUPPORTED and "vocab" in str(e.value)


def _step_bufs(n, Bn):
    return dict(canvas_out=torch.empty(n, dtype=torch.int32, device="cuda"),
                argmax_out=torch.empty(n, dtype=torch.int32, device="cuda"),
                sample_out=torch.empty(n, dtype=torch.int32, device="cuda"),
                accept_out=torch.empty(n, dtype=torch.uint8, device="cuda"),
                entropy_out=torch.empty(n, device="cuda"),
                n_accept_out=torch.empty(Bn, dtype=torch.int32, device="cuda"),
                mean_entropy_out=torch.empty(Bn, device="cuda"),
                stop_out=torch.empty(Bn, dtype=torch.uint8, device="cuda"))


def _workspace(ctx, Bn):
    return torch.empty(ctx.dg_lmhead_workspace_bytes(Bn), dtype=torch.uint8, device="cuda")


def _host_bufs(bufs):
    return {k: v.cpu().numpy() for k, v in bufs.items()}


def _canvas_outputs(g, c, L):
    rows = slice(c * L, (c + 1) * L)
    return dict(entropy=g["entropy_out"][rows], argmax=g["argmax_out"][rows], sample=g["sample_out"][rows],
                accept=g["accept_out"][rows], n_accept=g["n_accept_out"][c], canvas=g["canvas_out"][rows],
                mean_entropy=g["mean_entropy_out"][c], stop=g["stop_out"][c])


@pytest.mark.parametrize("L,Bn,K,V", [(256, 2, 128, 32768), (100, 3, 64, 8488), (16, 1, 64, 4104),
                                      (256, 1, 192, 262144)])
def test_fused_step_matches_oracle_on_its_product(L, Bn, K, V):
    # The fused step sees the product's fp32 logits bit for bit (the main loop
    # is shared with dg_lmhead_logits), so the oracle runs on those logits and
    # the comparison is the sampler's own: argmax identical, entropy within
    # H_TOL, samples equal except at near-ties. Shapes: whole tiles; 300 rows
    # (a ragged row tile) with V = 2 * 4096 + 296 (a chunk cut inside its first
    # stripe, so tiles past V hold no ids); a 16-row canvas with one id past a
    # chunk; the full 262144-id vocabulary.
    from full_parity import Tally, compare_step
    from oracle import parallel as OPAR
    require_gpu()
    params = B.params_default(canvas_len=L, vocab=V)
    ctx = B.Context(params, max_batch=Bn)
    h, w = synth.lmhead_operands(77 + V, Bn * L, K, V, device="cuda")
    temps_l = [0.8, 0.55, 0.4][:Bn]
    seeds_l = [5, 2**63 + 9, 77][:Bn]
    temps = torch.tensor(temps_l, device="cuda")
    seeds = seeds_tensor(seeds_l)
    z = torch.empty(Bn * L, V, device="cuda")
    ctx.dg_lmhead_logits(h, w, z)
    bufs = _step_bufs(Bn * L, Bn)
    ctx.dg_lmhead_sampler_step(h, w, _workspace(ctx, Bn), temps, 3, seeds, ctx.step_out(**bufs))
    # the plain step on the stored product: the same argmax bit for bit
    plain = _step_bufs(Bn * L, Bn)
    ctx.dg_sampler_step(z, temps, 3, seeds, ctx.step_out(**plain))
    torch.cuda.synchronize()
    g = _host_bufs(bufs)
    assert np.array_equal(g["argmax_out"], plain["argmax_out"].cpu().numpy())
    zh = z.cpu().numpy()
    _check_logits(zh, _f32(h), _f32(w), f"{Bn}x{L} rows, K {K}, V {V}")
    tally = Tally(f"fused {L}x{Bn} V{V}")
    jobs = [dict(rows=lambda r0, r1, c=c: zh[c * L + r0:c * L + r1].astype(np.float64), L=L, V=V,
                 temp=np.float32(temps_l[c]), seed=seeds_l[c], step=3, prev_argmax=None) for c in range(Bn)]
    for c, o in enumerate(OPAR.steps(jobs)):
        compare_step(_canvas_outputs(g, c, L), o, f"canvas {c}", tally, np.float32(0.1), np.float32(0.005))
    tally.report()


def test_fused_step_per_canvas_steps_deterministic_and_inactive():
    # per-canvas steps equal to the common step change nothing, a second call
    # gives the same bits (the per-row running best only lets tiles skip
    # draws that cannot win), and an inactive canvas's outputs stay untouched
    # while the others keep their values
    require_gpu()
    L, K, V, Bn = 256, 128, 32768, 3
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V), max_batch=Bn)
    h, w = synth.lmhead_operands(78, Bn * L, K, V, device="cuda")
    temps = torch.tensor([0.8, 0.55, 0.7], device="cuda")
    seeds = seeds_tensor([5, 2**63 + 9, 11])
    ws = _workspace(ctx, Bn)
    a = _step_bufs(Bn * L, Bn)
    ctx.dg_lmhead_sampler_step(h, w, ws, temps, 3, seeds, ctx.step_out(**a))
    b = _step_bufs(Bn * L, Bn)
    ctx.dg_lmhead_sampler_step(h, w, ws, temps, 0, seeds, ctx.step_out(**b),
                               steps=torch.tensor([3, 3, 3], dtype=torch.int32, device="cuda"))
    c = {k: torch.full_like(v, -5 if v.dtype == torch.int32 else 7) for k, v in _step_bufs(Bn * L, Bn).items()}
    ctx.dg_lmhead_sampler_step(h, w, ws, temps, 3, seeds, ctx.step_out(**c),
                               active=torch.tensor([1, 0, 1], dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key
    rows = slice(L, 2 * L)
    for key in ("canvas_out", "argmax_out", "sample_out", "accept_out", "entropy_out"):
        assert torch.all(c[key][rows] == (-5 if c[key].dtype == torch.int32 else 7)), key
        for keep in (slice(0, L), slice(2 * L, 3 * L)):
            assert torch.equal(c[key][keep], a[key][keep]), key
    for key in ("n_accept_out", "mean_entropy_out", "stop_out"):
        assert c[key][1].item() == (-5 if c[key].dtype == torch.int32 else 7), key
        assert c[key][0].item() == a[key][0].item() and c[key][2].item() == a[key][2].item(), key


def test_fused_lmhead_workload_matches_oracle():
    # 64 canvases x 256 positions, hidden bf16 [16384, 2048] ~ N(0,1), weight
    # bf16 [2048, 262144] ~ N(0, 1/2048); canvas c sits at step c mod 48 of the
    # default 48-step schedule (temperature and random draws), seed c. The
    # product's logits never leave the fused kernel; dg_lmhead_logits stores
    # the same product for the check. For eight canvases spread over the batch
    # every logit is checked against the oracle's exact product (within the
    # accumulation bound) and the oracle recomputes every row's statistics and
    # the canvas decisions on the product's logits; 8 rows of other canvases
    # are sampled the same way.
    from full_parity import Tally, compare_step
    from oracle import parallel as OPAR
    require_gpu()
    L, K, V, Bn = 256, 2048, 262144, 64
    params = B.params_default(canvas_len=L, vocab=V)
    ctx = B.Context(params, max_batch=Bn)
    h, w = synth.lmhead_operands(1005, Bn * L, K, V, device="cuda")
    steps = [c % 48 for c in range(Bn)]
    temps = [B.dg_temperature(params, s) for s in steps]
    seeds = list(range(Bn))
    ws = _workspace(ctx, Bn)
    assert ws.numel() == Bn * L * (16 * V // 4096) * 40 + Bn * L * 4
    bufs = _step_bufs(Bn * L, Bn)
    ctx.dg_lmhead_sampler_step(h, w, ws, torch.tensor(temps, device="cuda"), 0, seeds_tensor(seeds),
                               ctx.step_out(**bufs),
                               steps=torch.tensor(steps, dtype=torch.int32, device="cuda"))
    del ws
    z = torch.empty(Bn * L, V, device="cuda")
    ctx.dg_lmhead_logits(h, w, z)
    torch.cuda.synchronize()
    g = _host_bufs(bufs)
    wh = _f32(w)
    hh = _f32(h)
    tally = Tally("C5")
    for c in (0, 9, 18, 27, 36, 45, 54, 63):
        rows = slice(c * L, (c + 1) * L)
        t = np.float32(temps[c])
        assert t == np.float32(O.temperature(steps[c], 0.8, 0.4, 48))
        gz = z[c * L:(c + 1) * L].cpu().numpy()
        _check_logits(gz, hh[rows], wh, f"canvas {c} logits")
        o = OPAR.steps([dict(rows=lambda r0, r1: gz[r0:r1].astype(np.float64), L=L, V=V, temp=t, seed=c,
                             step=steps[c], prev_argmax=None)])[0]
        gc = _canvas_outputs(g, c, L)
        compare_step(gc, o, f"C5 canvas {c} (step {steps[c]})", tally, np.float32(0.1), np.float32(0.005))
        check_decision_rules(g["entropy_out"][rows], g["accept_out"][rows], g["n_accept_out"][c],
                             g["sample_out"][rows], g["canvas_out"][rows], o["renoise"],
                             g["mean_entropy_out"][c], g["stop_out"][c], None, g["argmax_out"][rows],
                             float(np.float32(0.1)), float(np.float32(0.005)))
        assert g["stop_out"][c] == 0
        print(f"canvas {c}: step {steps[c]} T {t:.4f} n_accept {g['n_accept_out'][c]} "
              f"(oracle {o['n_accept']})")
        del gz
    tally.report()
    report = []
    rng = np.random.default_rng(5)
    for r in rng.choice(np.arange(L, 63 * L), size=8, replace=False):
        c, pos = divmod(int(r), L)
        t = np.float32(temps[c])
        zr = z[r:r + 1].cpu().numpy()
        _check_logits(zr, hh[r:r + 1], wh, f"row {r} logits")
        compare_stats(zr.astype(np.float64), t, c, np.array([pos]), steps[c], g["entropy_out"][r:r + 1],
                      g["argmax_out"][r:r + 1], g["sample_out"][r:r + 1], report)
    print("sampled rows of other canvases:", report)


def test_lmhead_validation_rejects_before_launch():
    # every argument is checked before anything is enqueued: the logits
    # buffer keeps its sentinel after each rejected call
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=4, vocab=1024), max_batch=2)
    h, w = synth.lmhead_operands(3, 8, 64, 1024, device="cuda")
    z = torch.full((8, 1024), -7.0, device="cuda")
    L = B.lib()
    cases = [
        (lambda: L.dg_lmhead_logits(ctx.handle, 0, B._ptr(h), B._ptr(w), 64, B._ptr(z), 1024, None),
         B.DG_ERR_INVALID_ARG, "rows"),
        (lambda: L.dg_lmhead_logits(ctx.handle, 8, None, B._ptr(w), 64, B._ptr(z), 1024, None),
         B.DG_ERR_INVALID_ARG, "hidden"),
        (lambda: L.dg_lmhead_logits(ctx.handle, 8, B._ptr(h), None, 64, B._ptr(z), 1024, None),
         B.DG_ERR_INVALID_ARG, "weight"),
        (lambda: L.dg_lmhead_logits(ctx.handle, 8, B._ptr(h), B._ptr(w), 64, None, 1024, None),
         B.DG_ERR_INVALID_ARG, "logits"),
        (lambda: L.dg_lmhead_logits(ctx.handle, 8, B._ptr(h), B._ptr(w), 64, B._ptr(z), 1000, None),
         B.DG_ERR_INVALID_ARG, "ld_logits"),
        (lambda: L.dg_lmhead_logits(ctx.handle, 8, B._ptr(h[:, 1:]), B._ptr(w), 64, B._ptr(z), 1024, None),
         B.DG_ERR_UNSUPPORTED, "aligned"),
        (lambda: L.dg_lmhead_logits(ctx.handle, 8, B._ptr(h), B._ptr(w), 64, B._ptr(z), 1026, None),
         B.DG_ERR_UNSUPPORTED, "ld_logits"),
    ]
    for call, status, word in cases:
        assert call() == status
        assert word in L.dg_last_error(ctx.handle).decode()
    # the fused step checks its batch, step and workspace too; the workspace
    # keeps its sentinel after each rejected call
    seeds = seeds_tensor([1, 2])
    temps = torch.tensor([0.8, 0.8], device="cuda")
    canvas = torch.empty(8, dtype=torch.int32, device="cuda")
    need = ctx.dg_lmhead_workspace_bytes(2)
    assert need == 8 * 16 * 40 + 8 * 4
    ws = torch.full((need + 16,), 0xA5, dtype=torch.uint8, device="cuda")
    bad_calls = [
        (dict(step=-1), B.DG_ERR_INVALID_ARG, "step"),
        (dict(seeds=seeds_tensor([1, 2, 3])), B.DG_ERR_INVALID_ARG, "B = 3"),
        (dict(workspace=ws[:need - 4]), B.DG_ERR_INVALID_ARG, "workspace_bytes"),
        (dict(workspace=ws[1:need + 1]), B.DG_ERR_UNSUPPORTED, "workspace"),
        (dict(hidden=h[:, 1:]), B.DG_ERR_UNSUPPORTED, "hidden_dim"),
    ]
    for change, status, word in bad_calls:
        args = dict(hidden=h, workspace=ws[:need], step=0, seeds=seeds)
        args.update(change)
        with pytest.raises(B.DgError) as e:
            ctx.dg_lmhead_sampler_step(args["hidden"], w, args["workspace"], temps, args["step"], args["seeds"],
                                       ctx.step_out(canvas))
        assert e.value.status == status and word in str(e.value), (change, str(e.value))
    assert L.dg_lmhead_sampler_step(ctx.handle, 2, B._ptr(h), B._ptr(w), 64, None, need, B._ptr(temps), 0,
                                    None, B._ptr(seeds), None, None, ctypes.byref(ctx.step_out(canvas)),
                                    None) == B.DG_ERR_INVALID_ARG
    assert "workspace" in L.dg_last_error(ctx.handle).decode()
    with pytest.raises(B.DgError) as e:
        ctx.dg_lmhead_workspace_bytes(3)
    assert e.value.status == B.DG_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert torch.all(z == -7.0)
    assert torch.all(ws == 0xA5)
