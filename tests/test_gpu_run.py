"""GPU tests of the whole denoising loop (dg_run_canvas) and of multi-step
trajectories, against the oracle and against the properties the method has."""
import math

import numpy as np
import pytest
import torch

from canvas_sampler_amd import binding as B
from canvas_sampler_amd import synth
from oracle import philox as OP
from oracle import sampler as O

from gpu_util import check_decision_rules, compare_stats, gpu, host_values, require_gpu, seeds_tensor

pytestmark = gpu


def _sharpening_denoiser(gen_seeds, L, V, m0_max, dtype):
    def denoise(step, canvas_ptr, active_ptr, logits, stream):
        for c, g in enumerate(gen_seeds):
            synth.sharpening_logits(g, step, L, V, m0_max=m0_max, dtype=dtype, device="cuda",
                                    out=logits[c * L:(c + 1) * L])
    return denoise


def _run_gpu(ctx, seeds, denoise, dtype, record_canvas=False):
    Bn, L, V = len(seeds), ctx.L, ctx.V
    logits = torch.empty(Bn * L, V, dtype=dtype, device="cuda")
    final = torch.full((Bn, L), -1, dtype=torch.int32, device="cuda")
    canvases = []

    def wrapped(step, canvas_ptr, active_ptr, lg, stream):
        if record_canvas:
            buf = torch.empty(Bn, L, dtype=torch.int32, device="cuda")
            B.copy_from_device(buf, canvas_ptr)
            canvases.append(buf)
        denoise(step, canvas_ptr, active_ptr, lg, stream)

    steps, stopped = ctx.dg_run_canvas(seeds, wrapped, logits, final)
    torch.cuda.synchronize()
    return final.cpu().numpy(), steps, stopped, [c.cpu().numpy() for c in canvases]


def test_run_matches_oracle_trajectory_reduced_vocab():
    # sharpening denoiser (N(0,1) + m0 + 1.5*step at a fixed target, m0 ~ U[0,6]),
    # T 0.8 -> 0.4 over 16 steps, b = 0.1, cap 48; three canvases; V reduced so
    # that the oracle reruns every step in seconds
    L, V = 256, 16384
    gens = [1002, 2002, 3002]
    seeds = [0, 7, 2**63 + 5]
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V, temp_steps=16), max_batch=3)
    final, steps, stopped, canvases = _run_gpu(
        ctx, seeds, _sharpening_denoiser(gens, L, V, 6.0, torch.bfloat16), torch.bfloat16,
        record_canvas=True)
    for c in range(3):
        zs = {}

        def den(s, canvas, g=gens[c]):
            z = synth.sharpening_logits(g, s, L, V, m0_max=6.0, dtype=torch.bfloat16,
                                        device="cuda")
            zs[s] = z
            return host_values(z)

        ofinal, osteps, ostopped, rec = O.run(den, seeds[c], L, V, n_sched=16, record=True)
        # canvases handed to the denoiser: init canvas, then the renoised ones
        n = min(osteps, steps[c])
        diverged = None
        for s in range(n):
            if not np.array_equal(canvases[s][c], rec[s]["canvas_in"]):
                diverged = s
                break
        if diverged is None:
            assert steps[c] == osteps and stopped[c] == ostopped
            assert np.array_equal(final[c], ofinal)
            assert 2 <= osteps < 48
            print(f"canvas {c}: stopped after {osteps} steps, trajectory identical")
            continue
        # the trajectories may part only at a near-tie of the step before
        s = diverged - 1
        why = _explain_divergence(zs[s], rec[s], seeds[c], s, L, V, canvases[diverged][c])
        print(f"canvas {c}: trajectories part at step {diverged} through a near-tie ({why})")


def _explain_divergence(z, orec, seed, step, L, V, gpu_next_canvas):
    """Reruns step `step` on the GPU for one canvas and returns the near-tie
    that makes its next canvas differ from the oracle's; fails otherwise."""
    from gpu_util import accept_near_tie, near_tie
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V, temp_steps=16), max_batch=1)
    t = np.float32(O.temperature(step, 0.8, 0.4, 16))
    bufs = dict(canvas_out=torch.empty(L, dtype=torch.int32, device="cuda"),
                argmax_out=torch.empty(L, dtype=torch.int32, device="cuda"),
                sample_out=torch.empty(L, dtype=torch.int32, device="cuda"),
                accept_out=torch.empty(L, dtype=torch.uint8, device="cuda"),
                entropy_out=torch.empty(L, device="cuda"),
                n_accept_out=torch.empty(1, dtype=torch.int32, device="cuda"),
                mean_entropy_out=torch.empty(1, device="cuda"),
                stop_out=torch.empty(1, dtype=torch.uint8, device="cuda"))
    ctx.dg_sampler_step(z, torch.tensor([t], device="cuda"), step, seeds_tensor([seed]),
                        ctx.step_out(**bufs))
    torch.cuda.synchronize()
    g = {k: v.cpu().numpy() for k, v in bufs.items()}
    h, smp, mask = g["entropy_out"], g["sample_out"], g["accept_out"].astype(bool)
    zh = host_values(z)
    _, bbest, bgap, ebest, egap = O.sample_two_level_detail(zh, t, seed, np.arange(L), step)
    dh = float(np.max(np.abs(h - orec["entropy"])))
    ren = O.uniform_tokens(seed, L, step, V, OP.TAG_RENOISE)
    check_decision_rules(h, mask, g["n_accept_out"][0], smp, g["canvas_out"], ren,
                         g["mean_entropy_out"][0], g["stop_out"][0], None, g["argmax_out"],
                         float(np.float32(0.1)), float(np.float32(0.005)))
    assert np.array_equal(gpu_next_canvas, g["canvas_out"]), "rerun step differs from the run's"
    reasons = []
    bad = np.flatnonzero(smp != orec["sample"])
    ties = near_tie(bbest, bgap) | near_tie(ebest, egap)
    if np.any(mask[bad] | orec["accept"][bad]):
        hard = [i for i in bad if (mask[i] or orec["accept"][i]) and not ties[i]]
        assert not hard, f"sample differs at committed positions {hard} without a near-tie"
        reasons.append(f"sample near-tie at {list(bad)}")
    if not np.array_equal(mask, orec["accept"]):
        assert accept_near_tie(orec["entropy"], float(np.float32(0.1)), dh), \
            f"acceptance differs without a near-tie (max |dH| {dh:.2e})"
        reasons.append(f"acceptance boundary near-tie, max |dH| {dh:.2e}")
    assert reasons, "trajectories part without any difference at the step before"
    return "; ".join(reasons)


def test_exp_b_growth_sweep_matches_oracle():
    # "DiffusionGemma Lab" EXP B: the confidence-growth rate scaled by
    # 0.5/1/2/4 (sharpening margin growth 0.75/1.5/3/6 per step). Each run
    # through dg_run_canvas must stop where the oracle's does, with the same
    # final argmax canvas (or part from it only at a near-tie), and faster
    # growth must need fewer steps. V is reduced so the oracle runs in seconds.
    L, V = 256, 4096
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V, temp_steps=16), max_batch=1)
    gpu_steps = []
    for growth in (0.75, 1.5, 3.0, 6.0):
        def den_gpu(step, canvas_ptr, active_ptr, logits, stream, g=growth):
            synth.sharpening_logits(1002, step, L, V, m0_max=6.0, growth=g, dtype=torch.bfloat16,
                                    device="cuda", out=logits)
        final, steps, stopped, canvases = _run_gpu(ctx, [0], den_gpu, torch.bfloat16, record_canvas=True)
        zs = {}

        def den(s, canvas, g=growth):
            zs[s] = synth.sharpening_logits(1002, s, L, V, m0_max=6.0, growth=g, dtype=torch.bfloat16,
                                            device="cuda")
            return host_values(zs[s])

        ofinal, osteps, ostopped, rec = O.run(den, 0, L, V, n_sched=16, record=True)
        parted = next((s for s in range(min(osteps, steps[0]))
                       if not np.array_equal(canvases[s][0], rec[s]["canvas_in"])), None)
        if parted is None:
            assert stopped[0] == ostopped == 1
            assert steps[0] == osteps, f"growth {growth}: {steps[0]} steps, oracle {osteps}"
            assert np.array_equal(final[0], ofinal)
            print(f"growth {growth}: stops after {steps[0]} steps, as the oracle")
        else:
            why = _explain_divergence(zs[parted - 1], rec[parted - 1], 0, parted - 1, L, V, canvases[parted][0])
            print(f"growth {growth}: {steps[0]} steps (oracle {osteps}); parts at step {parted} ({why})")
        gpu_steps.append(steps[0])
    assert all(a >= b for a, b in zip(gpu_steps, gpu_steps[1:])) and gpu_steps[0] > gpu_steps[-1]


def test_exp_b_bound_sweep_commits_match_oracle():
    # "DiffusionGemma Lab" EXP B: raising the entropy bound raises the commits
    # per step. The sharpening denoiser is open loop (its logits do not depend
    # on the canvas), so every step can be compared with the oracle's on the
    # same logits: the commit count must agree (or sit at an acceptance near-tie)
    # and the mean commits per step must grow with the bound.
    from gpu_util import accept_near_tie
    L, V, steps = 256, 4096, 12
    require_gpu()
    means = []
    for bound in (0.01, 0.1, 1.0, 10.0):
        ctx = B.Context(B.params_default(canvas_len=L, vocab=V, temp_steps=16, entropy_bound=bound),
                        max_batch=1)
        bufs = dict(canvas_out=torch.empty(L, dtype=torch.int32, device="cuda"),
                    entropy_out=torch.empty(L, device="cuda"),
                    n_accept_out=torch.empty(1, dtype=torch.int32, device="cuda"))
        counts = []
        for s in range(steps):
            z = synth.sharpening_logits(1002, s, L, V, m0_max=6.0, dtype=torch.bfloat16, device="cuda")
            t = np.float32(O.temperature(s, 0.8, 0.4, 16))
            ctx.dg_sampler_step(z, torch.tensor([t], device="cuda"), s, seeds_tensor([0]),
                                ctx.step_out(**bufs))
            torch.cuda.synchronize()
            k = int(bufs["n_accept_out"].item())
            orec = O.step(host_values(z), t, 0, s, bound=np.float32(bound))
            if k != orec["n_accept"]:
                dh = float(np.max(np.abs(bufs["entropy_out"].cpu().numpy() - orec["entropy"])))
                assert accept_near_tie(orec["entropy"], float(np.float32(bound)), dh), \
                    f"bound {bound} step {s}: {k} commits, oracle {orec['n_accept']}"
            counts.append(k)
        means.append(float(np.mean(counts)))
        print(f"bound {bound}: {means[-1]:.1f} commits per step over {steps} steps")
    assert all(a <= b for a, b in zip(means, means[1:])) and means[0] < means[-1]


def test_full_vocab_steps_sampled_rows_and_exact_decisions():
    # the benchmark's single-canvas shape (B=1, 256 x 262144 bf16, nsplit auto),
    # stepped from Python so every step's outputs are visible: oracle statistics
    # on sampled rows, decisions checked exactly from the GPU's own entropies
    L, V = 256, 262144
    require_gpu()
    params = B.params_default(canvas_len=L, vocab=V, temp_steps=16)
    ctx = B.Context(params, max_batch=1)
    rows = np.array([0, 5, 64, 127, 200, 255])
    seeds = seeds_tensor([0])
    prev = None
    outs = {k: torch.empty(L, dtype=d, device="cuda") for k, d in
            (("canvas_out", torch.int32), ("sample_out", torch.int32), ("accept_out", torch.uint8),
             ("entropy_out", torch.float32))}
    am = [torch.empty(L, dtype=torch.int32, device="cuda") for _ in range(2)]
    nacc = torch.empty(1, dtype=torch.int32, device="cuda")
    meanh = torch.empty(1, device="cuda")
    stop = torch.empty(1, dtype=torch.uint8, device="cuda")
    stopped_at = None
    for s in range(48):
        z = synth.sharpening_logits(1002, s, L, V, m0_max=6.0, dtype=torch.bfloat16, device="cuda")
        t = B.dg_temperature(params, s)
        out = ctx.step_out(argmax_out=am[s & 1], n_accept_out=nacc, mean_entropy_out=meanh,
                           stop_out=stop, **outs)
        ctx.dg_sampler_step(z, torch.tensor([t], device="cuda"), s, seeds, out,
                            prev_argmax=None if s == 0 else am[(s + 1) & 1])
        torch.cuda.synchronize()
        g = {k: v.cpu().numpy() for k, v in outs.items()}
        gam = am[s & 1].cpu().numpy()
        zh = host_values(z[torch.as_tensor(rows, device="cuda")])
        compare_stats(zh, np.float32(t), 0, rows, s, g["entropy_out"][rows], gam[rows],
                      g["sample_out"][rows])
        ren = O.uniform_tokens(0, L, s, V, OP.TAG_RENOISE)
        check_decision_rules(g["entropy_out"], g["accept_out"], nacc.item(), g["sample_out"],
                             g["canvas_out"], ren, meanh.item(), stop.item(), prev, gam,
                             float(np.float32(0.1)), float(np.float32(0.005)))
        prev = gam
        if stop.item():
            stopped_at = s + 1
            break
    assert stopped_at is not None and stopped_at >= 2
    print("full-vocab sharpening canvas stopped after", stopped_at, "steps")


def test_batch_invariance_sixteen_canvases():
    # a canvas's trajectory depends only on its own seed and logits, not on the
    # batch it runs in: B=16 run vs single-canvas runs (full vocabulary, bf16)
    L, V, Bn = 256, 262144, 16
    require_gpu()
    params = B.params_default(canvas_len=L, vocab=V, temp_steps=48)
    gens = [(1003 << 32) | c for c in range(Bn)]
    seeds = list(range(Bn))
    ctx = B.Context(params, max_batch=Bn)
    final, steps, stopped, _ = _run_gpu(ctx, seeds,
                                        _sharpening_denoiser(gens, L, V, 8.0, torch.bfloat16),
                                        torch.bfloat16)
    assert all(stopped) and len(set(steps)) >= 1
    ctx1 = B.Context(params, max_batch=1)
    for c in (0, 5, 15):
        f1, s1, st1, _ = _run_gpu(ctx1, [seeds[c]],
                                  _sharpening_denoiser([gens[c]], L, V, 8.0, torch.bfloat16),
                                  torch.bfloat16)
        assert s1[0] == steps[c] and st1[0] == stopped[c]
        assert np.array_equal(f1[0], final[c])
    print("B=16 steps to stop:", steps)


def test_run_is_deterministic():
    L, V = 256, 32768
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V, temp_steps=16), max_batch=2)
    den = _sharpening_denoiser([11, 12], L, V, 6.0, torch.bfloat16)
    a = _run_gpu(ctx, [3, 4], den, torch.bfloat16)
    b = _run_gpu(ctx, [3, 4], den, torch.bfloat16)
    assert np.array_equal(a[0], b[0]) and a[1] == b[1] and a[2] == b[2]


def test_low_confidence_fp32_commits_one_per_step_to_cap():
    # untrained-model stand-in: iid N(0, 0.05) fp32 logits at V = 262144,
    # default schedule; exactly one commit per step, no stop before the cap
    L, V = 256, 262144
    require_gpu()
    params = B.params_default(canvas_len=L, vocab=V)
    ctx = B.Context(params, max_batch=1)
    seeds = seeds_tensor([0])
    canvas = torch.empty(L, dtype=torch.int32, device="cuda")
    ent = torch.empty(L, device="cuda")
    smp = torch.empty(L, dtype=torch.int32, device="cuda")
    am = [torch.empty(L, dtype=torch.int32, device="cuda") for _ in range(2)]
    nacc = torch.empty(1, dtype=torch.int32, device="cuda")
    stop = torch.empty(1, dtype=torch.uint8, device="cuda")
    rows = np.array([0, 99, 255])
    for s in range(48):
        z = synth.iid_normal_logits(1004, s, L, V, variance=0.05, dtype=torch.float32, device="cuda")
        t = B.dg_temperature(params, s)
        out = ctx.step_out(canvas, argmax_out=am[s & 1], sample_out=smp, entropy_out=ent,
                           n_accept_out=nacc, stop_out=stop)
        ctx.dg_sampler_step(z, torch.tensor([t], device="cuda"), s, seeds, out,
                            prev_argmax=None if s == 0 else am[(s + 1) & 1])
        torch.cuda.synchronize()
        assert nacc.item() == 1 and stop.item() == 0
        h = ent.cpu().numpy()
        assert abs(h.mean() - (math.log(V) - 0.05 / (2 * t * t))) < 0.03
        if s in (0, 23, 47):
            zh = host_values(z[torch.as_tensor(rows, device="cuda")])
            compare_stats(zh, np.float32(t), 0, rows, s, h[rows],
                          am[s & 1].cpu().numpy()[rows], smp.cpu().numpy()[rows])
    # and through the library loop: runs to the cap without stopping
    logits = torch.empty(L, V, device="cuda")
    final = torch.empty(1, L, dtype=torch.int32, device="cuda")

    def den(step, cp, ap, lg, stream):
        synth.iid_normal_logits(1004, step, L, V, variance=0.05, device="cuda", out=lg)

    steps, stopped = ctx.dg_run_canvas([0], den, logits, final)
    assert steps == [48] and stopped == [False]


def test_callback_failure_reports_and_keeps_steps():
    L, V = 64, 4096
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V), max_batch=1)
    logits = torch.empty(L, V, device="cuda")
    final = torch.empty(1, L, dtype=torch.int32, device="cuda")

    class Boom(RuntimeError):
        pass

    def den(step, cp, ap, lg, stream):
        if step == 3:
            raise Boom("denoiser failed")
        synth.iid_normal_logits(5, step, L, V, device="cuda", out=lg)

    with pytest.raises(Boom):
        ctx.dg_run_canvas([1], den, logits, final)
    # the library reported DG_ERR_CALLBACK; the context stays usable
    steps, stopped = ctx.dg_run_canvas(
        [1], lambda s, cp, ap, lg, st: synth.iid_normal_logits(5, s, L, V, device="cuda", out=lg),
        logits, final)
    assert steps == [48] and stopped == [False]


def _run_resident(ctx, seeds, denoise, dtype, check_every, record_canvas=False):
    """dg_run_canvas_resident with device seeds and outputs; the same return
    shape as _run_gpu."""
    Bn, L, V = len(seeds), ctx.L, ctx.V
    logits = torch.empty(Bn * L, V, dtype=dtype, device="cuda")
    final = torch.full((Bn, L), -1, dtype=torch.int32, device="cuda")
    steps = torch.full((Bn,), -1, dtype=torch.int32, device="cuda")
    stopped = torch.full((Bn,), 7, dtype=torch.uint8, device="cuda")
    canvases = []

    def wrapped(step, canvas_ptr, active_ptr, lg, stream):
        if record_canvas:
            buf = torch.empty(Bn, L, dtype=torch.int32, device="cuda")
            B.copy_from_device(buf, canvas_ptr)
            canvases.append(buf)
        denoise(step, canvas_ptr, active_ptr, lg, stream)

    ctx.dg_run_canvas_resident(seeds_tensor(seeds), wrapped, logits, final, steps, stopped,
                               check_every=check_every)
    torch.cuda.synchronize()
    return (final.cpu().numpy(), steps.cpu().tolist(), [bool(x) for x in stopped.cpu().tolist()],
            [c.cpu().numpy() for c in canvases])


def test_resident_run_matches_host_loop_and_oracle():
    # the device-resident loop (stop flags cleared on the device, no per-step
    # host wait) must give the host loop's results bit for bit, whether it
    # checks the flags every step, every 5 steps or never, and follow the
    # oracle's trajectories (or part from them only at a near-tie)
    L, V = 256, 16384
    gens = [1002, 2002, 3002]
    seeds = [0, 7, 2**63 + 5]
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V, temp_steps=16), max_batch=3)
    den = _sharpening_denoiser(gens, L, V, 6.0, torch.bfloat16)
    hfinal, hsteps, hstopped, _ = _run_gpu(ctx, seeds, den, torch.bfloat16)
    runs = {k: _run_resident(ctx, seeds, den, torch.bfloat16, k, record_canvas=(k == 0))
            for k in (0, 1, 5)}
    for k, (final, steps, stopped, _) in runs.items():
        assert steps == hsteps and stopped == hstopped, f"check_every {k}"
        assert np.array_equal(final, hfinal), f"check_every {k}"
    final, steps, stopped, canvases = runs[0]
    # with check_every 0 all 48 steps are enqueued; canvases that stopped
    # keep their state through the later (empty) steps
    assert len(canvases) == 48
    for c in range(3):
        zs = {}

        def oden(s, canvas, g=gens[c]):
            zs[s] = synth.sharpening_logits(g, s, L, V, m0_max=6.0, dtype=torch.bfloat16,
                                            device="cuda")
            return host_values(zs[s])

        ofinal, osteps, ostopped, rec = O.run(oden, seeds[c], L, V, n_sched=16, record=True)
        parted = next((s for s in range(min(osteps, steps[c]))
                       if not np.array_equal(canvases[s][c], rec[s]["canvas_in"])), None)
        if parted is None:
            assert steps[c] == osteps and stopped[c] == bool(ostopped)
            assert np.array_equal(final[c], ofinal)
            for s in range(osteps, 48):
                assert np.array_equal(canvases[s][c], canvases[osteps][c])
            print(f"canvas {c}: resident loop stops after {osteps} steps, as the oracle")
        else:
            why = _explain_divergence(zs[parted - 1], rec[parted - 1], seeds[c], parted - 1, L, V,
                                      canvases[parted][c])
            print(f"canvas {c}: parts from the oracle at step {parted} ({why})")


def test_resident_run_graph_replays():
    # the resident loop with check_every 0 waits for nothing, so the whole
    # run (denoiser included) is captured into one HIP graph; each replay,
    # with other work and a synchronisation between replays and new seeds
    # written into the device seed array, must equal an eager run
    L, V, Bn, cap = 256, 4096, 2, 24
    require_gpu()
    params = B.params_default(canvas_len=L, vocab=V, temp_steps=16, max_steps=cap)
    ctx = B.Context(params, max_batch=Bn)
    gens = [1002, 4002]
    pre = [torch.cat([synth.sharpening_logits(g, s, L, V, m0_max=6.0, dtype=torch.bfloat16,
                                              device="cuda") for g in gens]) for s in range(cap)]

    def den(step, canvas_ptr, active_ptr, lg, stream):
        lg.copy_(pre[step])

    eager = {}
    for seeds in ([0, 7], [123, 2**63 + 5]):
        r = _run_resident(ctx, seeds, den, torch.bfloat16, 0)
        h = _run_gpu(ctx, seeds, den, torch.bfloat16)
        assert r[1] == h[1] and r[2] == h[2] and np.array_equal(r[0], h[0])
        assert all(r[2]) and max(r[1]) < cap
        eager[tuple(seeds)] = r

    logits = torch.empty(Bn * L, V, dtype=torch.bfloat16, device="cuda")
    final = torch.empty(Bn, L, dtype=torch.int32, device="cuda")
    steps = torch.empty(Bn, dtype=torch.int32, device="cuda")
    stopped = torch.empty(Bn, dtype=torch.uint8, device="cuda")
    seeds_dev = seeds_tensor([0, 7])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ctx.dg_run_canvas_resident(seeds_dev, den, logits, final, steps, stopped, check_every=0)
    torch.cuda.synchronize()
    for seeds in ([0, 7], [123, 2**63 + 5], [0, 7], [123, 2**63 + 5]):
        seeds_dev.copy_(seeds_tensor(seeds))
        final.fill_(-1)
        steps.fill_(-1)
        stopped.fill_(9)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ef, es, est, _ = eager[tuple(seeds)]
        assert steps.cpu().tolist() == es
        assert [bool(x) for x in stopped.cpu().tolist()] == est
        assert np.array_equal(final.cpu().numpy(), ef)
    print("graph replays equal the eager runs; steps", {k: v[1] for k, v in eager.items()})


def test_resume_from_a_checkpoint_equals_the_uninterrupted_run():
    # the loop state between steps is the canvas, the previous argmax canvas
    # and the step index; a run stopped after step 3, its state copied to the
    # host, and continued on a fresh context must finish exactly like
    # dg_run_canvas (single canvas, sharpening stand-in, V = 16384)
    L, V, gen, seed = 256, 16384, 3002, 41
    require_gpu()
    params = B.params_default(canvas_len=L, vocab=V, temp_steps=16)
    den = _sharpening_denoiser([gen], L, V, 6.0, torch.bfloat16)
    final_ref, steps_ref, stopped_ref, _ = _run_gpu(B.Context(params, max_batch=1), [seed], den,
                                                    torch.bfloat16)

    def run_steps(ctx, canvas, prev, s0, s1):
        """Steps s0 .. s1-1 from (canvas, prev); returns the new state and
        (steps used, stopped) once the stop fires."""
        logits = torch.empty(L, V, dtype=torch.bfloat16, device="cuda")
        am = [torch.empty(L, dtype=torch.int32, device="cuda") for _ in range(2)]
        nxt = torch.empty(L, dtype=torch.int32, device="cuda")
        stop = torch.empty(1, dtype=torch.uint8, device="cuda")
        for s in range(s0, s1):
            synth.sharpening_logits(gen, s, L, V, m0_max=6.0, dtype=torch.bfloat16, device="cuda",
                                    out=logits)
            out = ctx.step_out(nxt, argmax_out=am[s & 1], stop_out=stop)
            t = torch.tensor([B.dg_temperature(params, s)], device="cuda")
            ctx.dg_sampler_step(logits, t, s, seeds_tensor([seed]), out, prev_argmax=prev)
            torch.cuda.synchronize()
            if stop.item():
                return nxt.clone(), am[s & 1].clone(), (s + 1, True)
            canvas, prev = nxt.clone(), am[s & 1].clone()
        return canvas, prev, None

    ctx = B.Context(params, max_batch=1)
    canvas = torch.empty(1, L, dtype=torch.int32, device="cuda")
    ctx.dg_canvas_init(seeds_tensor([seed]), canvas)
    canvas, prev, done = run_steps(ctx, canvas.view(-1), None, 0, 3)
    assert done is None
    saved = (canvas.cpu().numpy(), prev.cpu().numpy())
    ctx.close()
    del canvas, prev
    torch.cuda.synchronize()
    ctx2 = B.Context(params, max_batch=1)
    canvas = torch.as_tensor(saved[0], device="cuda")
    prev = torch.as_tensor(saved[1], device="cuda")
    _, final, done = run_steps(ctx2, canvas, prev, 3, 48)
    assert done is not None, "the resumed run did not stop"
    assert done == (steps_ref[0], stopped_ref[0])
    assert np.array_equal(final.cpu().numpy(), final_ref[0])
    print(f"resumed after 3 steps; stops after {done[0]} steps like the uninterrupted run")
