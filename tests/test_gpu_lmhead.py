"""GPU parity of the LM-head configuration (dg_lmhead_logits,
dg_lmhead_sampler_step) against the oracle's exact products, through the C ABI.

Logit tolerance. The GPU sums K bf16 products with fp32 accumulation on the
matrix cores (32 products per instruction, K/32 instructions chained). To
first order in u = 2^-24 the error of such a sum is at most
(K/32 + 31) * u * sum_k |h_k w_k|: at most 31 roundings inside one
instruction's 32-term sum, one per chained accumulation. Every logit is checked
against that bound; the measured maximum is printed (it is far smaller).
"""
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


def test_lmhead_step_equals_sampler_step_on_its_logits():
    # the fused entry point is the product followed by the plain step: same
    # kernels, so every output is identical; per-canvas steps equal to the
    # common step change nothing
    require_gpu()
    L, K, V, Bn = 256, 128, 32768, 2
    params = B.params_default(canvas_len=L, vocab=V)
    ctx = B.Context(params, max_batch=Bn)
    h, w = synth.lmhead_operands(77, Bn * L, K, V, device="cuda")
    temps = torch.tensor([0.8, 0.55], device="cuda")
    seeds = seeds_tensor([5, 2**63 + 9])
    z = torch.empty(Bn * L, V, device="cuda")
    a = _step_bufs(Bn * L, Bn)
    ctx.dg_lmhead_sampler_step(h, w, z, temps, 3, seeds, ctx.step_out(**a))
    b = _step_bufs(Bn * L, Bn)
    ctx.dg_sampler_step(z.clone(), temps, 3, seeds, ctx.step_out(**b))
    c = _step_bufs(Bn * L, Bn)
    ctx.dg_lmhead_sampler_step(h, w, torch.empty_like(z), temps, 0, seeds, ctx.step_out(**c),
                               steps=torch.tensor([3, 3], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key
        assert torch.equal(a[key], c[key]), key


def test_fused_lmhead_workload_matches_oracle():
    # 64 canvases x 256 positions, hidden bf16 [16384, 2048] ~ N(0,1), weight
    # bf16 [2048, 262144] ~ N(0, 1/2048); canvas c sits at step c mod 48 of the
    # default 48-step schedule (temperature and random draws), seed c. The
    # oracle recomputes eight canvases spread over the batch completely (every
    # logit within the accumulation bound, then every row's statistics and
    # the canvas decisions on the exact logits), plus 8 sampled rows of others.
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
    z = torch.empty(Bn * L, V, device="cuda")
    bufs = _step_bufs(Bn * L, Bn)
    ctx.dg_lmhead_sampler_step(h, w, z, torch.tensor(temps, device="cuda"), 0, seeds_tensor(seeds),
                               ctx.step_out(**bufs),
                               steps=torch.tensor(steps, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in bufs.items()}
    wh = _f32(w)
    hh = _f32(h)
    tally = Tally("C5")
    for c in (0, 9, 18, 27, 36, 45, 54, 63):
        rows = slice(c * L, (c + 1) * L)
        t = np.float32(temps[c])
        assert t == np.float32(O.temperature(steps[c], 0.8, 0.4, 48))
        exact = OL.logits(hh[rows], wh)
        gz = z[c * L:(c + 1) * L].cpu().numpy()
        _, err = _check_logits(gz, hh[rows], wh, f"canvas {c} logits", exact=exact)
        o = OPAR.steps([dict(rows=lambda r0, r1: exact[r0:r1], L=L, V=V, temp=t, seed=c, step=steps[c],
                             prev_argmax=None)])[0]
        gc = dict(entropy=g["entropy_out"][rows], argmax=g["argmax_out"][rows], sample=g["sample_out"][rows],
                  accept=g["accept_out"][rows], n_accept=g["n_accept_out"][c], canvas=g["canvas_out"][rows],
                  mean_entropy=g["mean_entropy_out"][c], stop=g["stop_out"][c])
        compare_step(gc, o, f"C5 canvas {c} (step {steps[c]})", tally, np.float32(0.1), np.float32(0.005),
                     logit_err=err.max(axis=1), z=exact, temp=t)
        check_decision_rules(g["entropy_out"][rows], g["accept_out"][rows], g["n_accept_out"][c],
                             g["sample_out"][rows], g["canvas_out"][rows], o["renoise"],
                             g["mean_entropy_out"][c], g["stop_out"][c], None, g["argmax_out"][rows],
                             float(np.float32(0.1)), float(np.float32(0.005)))
        assert g["stop_out"][c] == 0
        print(f"canvas {c}: step {steps[c]} T {t:.4f} n_accept {g['n_accept_out'][c]} "
              f"(oracle {o['n_accept']})")
        del exact, err
    tally.report()
    report = []
    rng = np.random.default_rng(5)
    for r in rng.choice(np.arange(L, 63 * L), size=8, replace=False):
        c, pos = divmod(int(r), L)
        t = np.float32(temps[c])
        zr = OL.logits(hh[r:r + 1], wh)
        _, err = _check_logits(z[r:r + 1].cpu().numpy(), hh[r:r + 1], wh, f"row {r} logits", exact=zr)
        compare_stats(zr, t, c, np.array([pos]), steps[c], g["entropy_out"][r:r + 1],
                      g["argmax_out"][r:r + 1], g["sample_out"][r:r + 1], report,
                      logit_err=err.max(axis=1))
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
    # the fused step checks its batch and step too
    seeds = seeds_tensor([1, 2])
    temps = torch.tensor([0.8, 0.8], device="cuda")
    canvas = torch.empty(8, dtype=torch.int32, device="cuda")
    with pytest.raises(B.DgError) as e:
        ctx.dg_lmhead_sampler_step(h, w, z, temps, -1, seeds, ctx.step_out(canvas))
    assert e.value.status == B.DG_ERR_INVALID_ARG and "step" in str(e.value)
    with pytest.raises(B.DgError) as e:
        ctx.dg_lmhead_sampler_step(h, w, z, temps, 0, seeds_tensor([1, 2, 3]), ctx.step_out(canvas))
    assert e.value.status == B.DG_ERR_INVALID_ARG and "B = 3" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(z == -7.0)
