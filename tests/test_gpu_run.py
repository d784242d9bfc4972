"""GPU tests of the whole denoising loop (dg_run_canvas) and of multi-step
trajectories, against the oracle and against the properties the method has."""
import numpy as np
import pytest
import torch

from canvas_sampler_amd import binding as B
from canvas_sampler_amd import synth

from full_parity import sharpening_writer, trajectory
from gpu_util import gpu, require_gpu, seeds_tensor

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
    # T 0.8 -> 0.4 over 16 steps, b = 0.1, cap 48; three canvases with their own
    # generator and sampler seeds (one of them above 2^63); V reduced so that
    # the canvases run in one batch at modest oracle cost. Every row of every
    # step against the oracle; dg_run_canvas must end where the steps did.
    L, V = 256, 16384
    require_gpu()
    tally, runs, _ = trajectory("sharpening V=16384 x3", L, V, [0, 7, 2**63 + 5],
                                sharpening_writer([1002, 2002, 3002], L, V, 6.0, torch.bfloat16),
                                torch.bfloat16, temp_steps=16)
    assert all(r[1] and 2 <= r[0] < 48 for r in runs)
    tally.report()


def test_exp_b_growth_sweep_matches_oracle():
    # "DiffusionGemma Lab" EXP B: the confidence-growth rate scaled by
    # 0.5/1/2/4 (sharpening margin growth 0.75/1.5/3/6 per step). Each run must
    # match the oracle's on every row of every step and stop where it does,
    # and faster growth must need fewer steps. V is reduced so the oracle runs
    # in seconds.
    L, V = 256, 4096
    require_gpu()
    gpu_steps = []
    for growth in (0.75, 1.5, 3.0, 6.0):
        tally, runs, _ = trajectory(f"EXP B growth {growth}", L, V, [0],
                                    sharpening_writer([1002], L, V, 6.0, torch.bfloat16, growth=growth),
                                    torch.bfloat16, temp_steps=16)
        assert runs[0][1]
        gpu_steps.append(runs[0][0])
        tally.report()
    assert all(a >= b for a, b in zip(gpu_steps, gpu_steps[1:])) and gpu_steps[0] > gpu_steps[-1]


def test_exp_b_bound_sweep_commits_match_oracle():
    # "DiffusionGemma Lab" EXP B: raising the entropy bound raises the commits
    # per step. Each bound's run matches the oracle on every row of every step
    # (acceptance differences only at counted near-ties) and the mean commits
    # per step must grow with the bound.
    L, V = 256, 4096
    require_gpu()
    means = []
    for bound in (0.01, 0.1, 1.0, 10.0):
        tally, runs, commits = trajectory(f"EXP B bound {bound}", L, V, [0],
                                          sharpening_writer([1002], L, V, 6.0, torch.bfloat16),
                                          torch.bfloat16, temp_steps=16, bound=bound)
        means.append(float(np.mean(commits[0])))
        print(f"bound {bound}: {means[-1]:.1f} commits per step over {runs[0][0]} steps")
        tally.report()
    assert all(a <= b for a, b in zip(means, means[1:])) and means[0] < means[-1]


def test_batch_invariance_sixteen_canvases():
    # a canvas's trajectory depends only on its own seed and logits, not on the
    # batch it runs in: B=16 run vs single-canvas runs (full vocabulary, bf16)
    L, V, Bn = 256, 262144, 16
    require_gpu()
    params = B.params_default(canvas_len=L, vocab=V, temp_steps=16)
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
    den_w = sharpening_writer(gens, L, V, 6.0, torch.bfloat16)
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
        for s_ in range(steps[c], 48):
            assert np.array_equal(canvases[s_][c], canvases[steps[c]][c])
    # the same canvases stepped from Python against the oracle, every row of
    # every step: the resident loop must end where they do
    tally, oruns, _ = trajectory("resident V=16384 x3", L, V, seeds, den_w, torch.bfloat16, temp_steps=16,
                                 library_loop=False)
    for c in range(3):
        assert (steps[c], stopped[c]) == oruns[c][:2]
        assert np.array_equal(final[c], oruns[c][2])
    tally.report()


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
