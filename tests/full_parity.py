"""Whole denoising runs compared with the oracle on every row of every step.

trajectory() steps B canvases through dg_sampler_step from Python, so every
step's outputs are visible, and runs the oracle (oracle.parallel: the oracle's
own per-row functions over a thread pool) on the very same logits bits for
every row of every canvas still running. It then checks that the library's
own loop (dg_run_canvas) ends exactly where the Python-driven steps did.

The synthetic denoisers are open loop: their logits depend on (seed, canvas,
step, position) only, never on the canvas. So each step's statistics, stop
decision and argmax canvas can be compared whatever happened at earlier
steps, and the steps used, the stop flag and the final argmax canvas of every
canvas must equal the oracle's even where a near-tie made one step's new
canvas differ ("DiffusionGemma Lab" §2 items 2, 3, 5; "DiffusionGemma:
Parallel Denoising From an Autoregressive Checkpoint", Finding, Algorithm 1).

Per row and step: |dH| <= 1e-4, argmax bit-exact, sample bit-exact except
counted sample near-ties. Per canvas and step: acceptance, new canvas and
stop exact except counted acceptance or stop near-ties, each named with the
slack that excused it (gpu_util.accept_tie_clause, stop_tie_clause).
Tally.report() prints the counts and, when DG_PARITY_DIR is set, writes them
as JSON into that directory.
"""
import json
import os
import time

import numpy as np
import torch

from canvas_sampler_amd import binding as B
from oracle import parallel as OPAR

from gpu_util import H_TOL, accept_tie_clause, near_tie, seeds_tensor, stop_tie_clause


class Tally:
    """Counts of one configuration's comparison with the oracle."""

    def __init__(self, name):
        self.name = name
        self.canvas_steps = 0
        self.rows = 0
        self.max_dh = 0.0
        self.near_tie_rows = 0        # rows whose oracle sample is a near-tie (either level)
        self.sample_near_ties = 0     # of those, rows where the GPU drew another id
        self.accept_near_ties = 0     # canvas steps whose acceptance differs at a near-tie
        self.stop_near_ties = 0
        self.argmax_near_ties = 0     # LM-head logits only: argmax within the logit error
        self.canvas_positions_differ = 0
        self.clauses = []
        self.trajectories = 0
        self.trajectories_equal = 0   # steps used, stop flag and final argmax canvas equal
        self.oracle_s = 0.0

    def record(self):
        return {"config": self.name, "canvas_steps": self.canvas_steps, "rows_compared": self.rows,
                "max_abs_dH": self.max_dh, "sample_near_tie_rows": self.near_tie_rows,
                "sample_mismatches_at_near_ties": self.sample_near_ties,
                "accept_near_ties": self.accept_near_ties, "stop_near_ties": self.stop_near_ties,
                "argmax_near_ties": self.argmax_near_ties,
                "canvas_positions_differing": self.canvas_positions_differ,
                "trajectories": self.trajectories, "trajectories_equal": self.trajectories_equal,
                "clauses": self.clauses[:20], "oracle_seconds": round(self.oracle_s, 2)}

    def report(self):
        rec = self.record()
        print("parity", json.dumps(rec), flush=True)
        out_dir = os.environ.get("DG_PARITY_DIR")
        if out_dir:
            os.makedirs(out_dir, exist_ok=True)
            with open(os.path.join(out_dir, self.name + ".json"), "w") as f:
                json.dump(rec, f, indent=1)
        return rec


def compare_step(g, o, label, tally, bound, threshold, logit_err=None, z=None, temp=None):
    """One canvas's GPU outputs of one step (g: host arrays) against the
    oracle's (o: oracle.parallel.steps record) on the same logits.

    When the GPU's logits are its own product (the LM head) rather than the
    oracle's input, logit_err gives each row's largest measured logit error
    and z the oracle's logits: an argmax difference is then a near-tie when the
    two logits lie within 2 * err of each other, and a sample difference when
    a Gumbel margin lies within 2 * err / T."""
    L = len(o["entropy"])
    h_g = np.asarray(g["entropy"], dtype=np.float64)
    dh = float(np.max(np.abs(h_g - o["entropy"])))
    assert dh <= H_TOL, f"{label}: entropy error {dh:.3g} > {H_TOL}"
    tally.canvas_steps += 1
    tally.rows += L
    tally.max_dh = max(tally.max_dh, dh)

    gam = np.asarray(g["argmax"])
    bad = np.flatnonzero(gam != o["argmax"])
    if logit_err is not None and bad.size:
        gap = z[bad, o["argmax"][bad]] - z[bad, gam[bad]]
        excused = gap <= 2 * logit_err[bad]
        tally.argmax_near_ties += int(excused.sum())
        bad = bad[~excused]
    assert bad.size == 0, f"{label}: argmax differs at rows {bad[:10]}"

    ties = near_tie(o["block_best"], o["block_gap"]) | near_tie(o["elem_best"], o["elem_gap"])
    if logit_err is not None:
        slack = 2 * logit_err / float(temp)
        ties = ties | (o["block_gap"] < slack) | (o["elem_gap"] < slack)
    mism = np.asarray(g["sample"]) != o["sample"]
    hard = np.flatnonzero(mism & ~ties)
    assert hard.size == 0, (f"{label}: sample differs at rows {hard[:10]} that are not near-ties "
                            f"(block gaps {o['block_gap'][hard[:5]]}, element gaps {o['elem_gap'][hard[:5]]})")
    tally.near_tie_rows += int(ties.sum())
    tally.sample_near_ties += int((mism & ties).sum())

    acc_g = np.asarray(g["accept"]).astype(bool)
    acc_o = o["accept"]
    if not np.array_equal(acc_g, acc_o) or int(g["n_accept"]) != int(o["n_accept"]):
        clause = accept_tie_clause(o["entropy"], float(bound), dh)
        assert clause, (f"{label}: acceptance differs ({int(g['n_accept'])} vs oracle {int(o['n_accept'])}) "
                        f"without a near-tie (max |dH| {dh:.3g})")
        tally.accept_near_ties += 1
        tally.clauses.append(f"{label}: acceptance {int(g['n_accept'])} vs {int(o['n_accept'])}: {clause}")

    canvas = np.asarray(g["canvas"])
    assert np.array_equal(canvas, np.where(acc_g, g["sample"], o["renoise"])), \
        f"{label}: the new canvas is not sample-where-accepted, renoise-elsewhere"
    same_inputs = (acc_g == acc_o) & (~acc_o | ~mism)
    assert np.array_equal(canvas[same_inputs], o["canvas"][same_inputs]), f"{label}: canvas differs"
    tally.canvas_positions_differ += int(np.sum(canvas != o["canvas"]))

    m_g = float(g["mean_entropy"])
    assert abs(m_g - o["mean_entropy"]) <= dh + 2.0 ** -22 * max(1.0, o["mean_entropy"]), \
        f"{label}: mean entropy {m_g} vs oracle {o['mean_entropy']}"
    if bool(g["stop"]) != bool(o["stop"]):
        clause = stop_tie_clause(o["mean_entropy"], threshold, dh)
        assert clause, f"{label}: stop {bool(g['stop'])} vs oracle {bool(o['stop'])} without a near-tie"
        tally.stop_near_ties += 1
        tally.clauses.append(f"{label}: stop: {clause}")
        return False
    return True


def _host_rows(t):
    """Host copy of a logits slab as float32 (bf16 and fp32 widen exactly)."""
    return t.to("cpu").to(torch.float32).numpy()


def trajectory(name, L, V, seeds, write_logits, dtype, temp_steps=48, bound=0.1, cap=48,
               tally=None, library_loop=True, on_step=None, log=print):
    """Runs len(seeds) canvases to their stop (or the cap) on the GPU and in
    the oracle, comparing every row of every step (see the module docstring).

    write_logits(step, out) must enqueue on the current stream the writing of
    every canvas's logits at `step` into out [B*L, V] (canvas c in rows
    c*L .. c*L+L-1); it is called again with the same step by dg_run_canvas.
    on_step(step, canvas, gpu, oracle), if given, sees each compared canvas
    step (host dicts). Returns (tally, per-canvas (steps used, stopped, final
    argmax canvas), per-canvas lists of the GPU's commits per step)."""
    n = len(seeds)
    tally = tally or Tally(name)
    params = B.params_default(canvas_len=L, vocab=V, temp_steps=temp_steps, entropy_bound=bound,
                              max_steps=cap)
    bound32 = np.float32(params.entropy_bound)
    thr32 = np.float32(params.stop_mean_entropy)
    ctx = B.Context(params, max_batch=n)
    dev = "cuda"
    logits = torch.empty(n * L, V, dtype=dtype, device=dev)
    bufs = dict(canvas_out=torch.empty(n * L, dtype=torch.int32, device=dev),
                sample_out=torch.empty(n * L, dtype=torch.int32, device=dev),
                accept_out=torch.empty(n * L, dtype=torch.uint8, device=dev),
                entropy_out=torch.empty(n * L, device=dev),
                n_accept_out=torch.empty(n, dtype=torch.int32, device=dev),
                mean_entropy_out=torch.empty(n, device=dev),
                stop_out=torch.empty(n, dtype=torch.uint8, device=dev))
    am = [torch.empty(n * L, dtype=torch.int32, device=dev) for _ in range(2)]
    active_dev = torch.ones(n, dtype=torch.uint8, device=dev)
    seeds_dev = seeds_tensor(seeds)
    g_run = [None] * n     # (steps used, stopped, final argmax) once finished
    o_run = [None] * n
    o_prev = [None] * n
    g_last = [None] * n
    o_last = [None] * n
    excused = set()
    commits = [[] for _ in range(n)]
    for s in range(cap):
        g_live = [c for c in range(n) if g_run[c] is None]
        o_live = [c for c in range(n) if o_run[c] is None]
        if not g_live and not o_live:
            break
        write_logits(s, logits)
        t = B.dg_temperature(params, s)
        out = ctx.step_out(argmax_out=am[s & 1], **bufs)
        # while every canvas runs, no active mask (the launch of the benchmark
        # lines, which takes the persistent row loop for large batches); the
        # mask once a canvas has stopped (the launch dg_run_canvas makes)
        ctx.dg_sampler_step(logits, torch.full((n,), t, device=dev), s, seeds_dev, out,
                            prev_argmax=am[(s + 1) & 1] if s else None,
                            active=None if len(g_live) == n else active_dev)
        torch.cuda.synchronize()
        g = {k: v.cpu().numpy() for k, v in bufs.items()}
        gam = am[s & 1].cpu().numpy()
        hosts = {c: _host_rows(logits[c * L:(c + 1) * L]) for c in o_live}
        jobs = [dict(rows=lambda r0, r1, zc=hosts[c]: zc[r0:r1], L=L, V=V, temp=np.float32(t),
                     seed=seeds[c], step=s, prev_argmax=o_prev[c]) for c in o_live]
        t0 = time.perf_counter()
        res = dict(zip(o_live, OPAR.steps(jobs, bound=bound32, stop_threshold=thr32)))
        tally.oracle_s += time.perf_counter() - t0
        del hosts, jobs
        for c in g_live:
            sl = slice(c * L, (c + 1) * L)
            gc = dict(entropy=g["entropy_out"][sl], argmax=gam[sl], sample=g["sample_out"][sl],
                      accept=g["accept_out"][sl], n_accept=g["n_accept_out"][c], canvas=g["canvas_out"][sl],
                      mean_entropy=g["mean_entropy_out"][c], stop=g["stop_out"][c])
            if c in res:
                if not compare_step(gc, res[c], f"{name} canvas {c} step {s}", tally, bound32, thr32):
                    excused.add(c)
                if on_step is not None:
                    on_step(s, c, gc, res[c])
            commits[c].append(int(gc["n_accept"]))
            g_last[c] = gc["argmax"].copy()
            if gc["stop"]:
                g_run[c] = (s + 1, True, g_last[c])
                active_dev[c] = 0
        for c in o_live:
            o_prev[c] = o_last[c] = res[c]["argmax"]
            if res[c]["stop"]:
                o_run[c] = (s + 1, True, o_last[c])
        log(f"{name} step {s}: canvases running {len(g_live)} (oracle {len(o_live)}), "
            f"commits {[int(g['n_accept_out'][c]) for c in g_live][:16]}, "
            f"oracle {tally.oracle_s:.1f} s so far", flush=True)
    for c in range(n):
        if g_run[c] is None:
            g_run[c] = (cap, False, g_last[c])
        if o_run[c] is None:
            o_run[c] = (cap, False, o_last[c])
        tally.trajectories += 1
        same = (g_run[c][0] == o_run[c][0] and g_run[c][1] == o_run[c][1]
                and np.array_equal(g_run[c][2], o_run[c][2]))
        if c not in excused:
            assert same, (f"{name} canvas {c}: GPU steps {g_run[c][0]} stopped {g_run[c][1]}, "
                          f"oracle steps {o_run[c][0]} stopped {o_run[c][1]}")
        tally.trajectories_equal += int(same)
    if library_loop:
        final = torch.full((n, L), -1, dtype=torch.int32, device=dev)

        def den(step, canvas_ptr, active_ptr, lg, stream):
            write_logits(step, lg)

        steps, stopped = ctx.dg_run_canvas(seeds, den, logits, final)
        torch.cuda.synchronize()
        fin = final.cpu().numpy()
        for c in range(n):
            assert (steps[c], stopped[c]) == g_run[c][:2], \
                f"{name} canvas {c}: dg_run_canvas {steps[c]}, {stopped[c]} vs stepped {g_run[c][:2]}"
            assert np.array_equal(fin[c], g_run[c][2]), f"{name} canvas {c}: dg_run_canvas final argmax differs"
    ctx.close()
    del logits
    torch.cuda.empty_cache()
    return tally, g_run, commits


def sharpening_writer(gens, L, V, m0_max, dtype, growth=1.5):
    """write_logits for the sharpening stand-in: canvas c draws from generator
    seed gens[c] (fixed targets and base margins m0 ~ U[0, m0_max]; fresh
    N(0,1) each step plus m0 + growth * step at the target)."""
    from canvas_sampler_amd import synth

    def write(step, out):
        for c, g in enumerate(gens):
            synth.sharpening_logits(g, step, L, V, m0_max=m0_max, growth=growth, dtype=dtype, device="cuda",
                                    out=out[c * L:(c + 1) * L])
    return write
