#!/usr/bin/env python3
"""Throughput of one canvas-sampler step on one MI355X.

A step is the whole per-step hot path on one batch of synthetic logits that
are already resident in HBM: the streaming statistics kernel (entropy, argmax,
two-level Gumbel-max sample per position) followed by the per-canvas
accept/renoise/stop kernel. Workload: one canvas of 256 positions, a
262,144-token vocabulary, bf16 logits from the sharpening denoiser; the logits
rotate over several 128 MiB buffers so that each step reads from HBM rather
than from the 256 MB last-level cache. Steps are launched back to back on one
stream (the host enqueues faster than the GPU drains, so host launch cost is
hidden); the same steps replayed from captured HIP graphs (one step per graph,
and one graph holding a step on each buffer) are reported too.

Prints one JSON line: steps/s (value), positions/s, the statistics kernel's
achieved HBM bandwidth against the 8 TB/s peak (HIP events on the launch
stream), the oracle's rate on the host cores with the agreement of every
configuration's sample with it ("parity"), and (under "lmhead") the step of
64 canvases whose logits come from the bf16 LM-head product, hidden
[16384, 2048] x weight [2048, 262144]: the product's time and matrix-core
throughput against the 2.5 PFLOP/s dense bf16 peak, and the whole step's time.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sampler steps/sec & canvas-positions/sec at 256xV=262144 bf16; % HBM peak"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "canvas_stats_traffic.json")
STATS_SRC = os.path.join(ROOT, "canvas_sampler_amd", "csrc", "canvas_stats.hip")


def _sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _traffic(bytes_per_launch):
    """HBM traffic per launch from the committed rocprofv3 counter summary,
    or None when there is none or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != _sha(STATS_SRC):
        return None
    return rec.get("hbm_bytes_per_launch")


def _oracle_canvas_worker(job):
    """One canvas's oracle step in a fresh process (no GPU): builds its
    logits on the CPU and returns the seconds O.step takes."""
    os.environ["HIP_VISIBLE_DEVICES"] = ""
    import numpy as np
    import torch
    torch.set_num_threads(1)
    from canvas_sampler_amd import synth
    from oracle import sampler as O
    gen, seed, L, V = job
    z = synth.sharpening_logits(gen, 0, L, V, m0_max=8.0, dtype=torch.bfloat16)
    zh = z.to(torch.float64).numpy()
    t0 = time.perf_counter()
    O.step(zh, np.float32(0.8), seed, 0)
    return time.perf_counter() - t0


def cpu_full_leg(workers):
    """The oracle's rates on the host for the configurations of the scope
    table: single steps of C1 (V = 4096 fp32), C2 (262144 bf16) and C4
    (262144 fp32 iid N(0, 0.05)) on one thread, the full C2 run (10 steps) on
    one thread, and one step of C3 (16 canvases of C2's shape) with one
    canvas per process over `workers` processes. The oracle handles one canvas
    at a time on one thread, so a single canvas gains nothing from more
    cores. Inputs come from the CPU generators (same shapes and
    distributions as the GPU runs)."""
    import multiprocessing as mp

    import numpy as np
    import torch

    from canvas_sampler_amd import synth
    from oracle import sampler as O

    torch.set_num_threads(1)
    L, V = 256, 262144
    out = {"threads_per_process": 1}

    def timed(fn, reps=1):
        best = None
        for _ in range(reps):
            t0 = time.perf_counter()
            fn()
            dt = time.perf_counter() - t0
            best = dt if best is None or dt < best else best
        return best

    z1 = synth.margin_logits(1001, L, 4096, m_max=12.0).to(torch.float64).numpy()
    t = timed(lambda: O.step(z1, np.float32(0.8), 0, 0), reps=3)
    out["c1_step_s"], out["c1_positions_per_s"] = t, L / t
    z2 = synth.sharpening_logits(1002, 0, L, V, m0_max=6.0, dtype=torch.bfloat16).to(torch.float64).numpy()
    t = timed(lambda: O.step(z2, np.float32(0.8), 0, 0), reps=2)
    out["c2_step_s"], out["c2_positions_per_s"] = t, L / t
    z4 = synth.iid_normal_logits(1004, 0, L, V, variance=0.05).to(torch.float64).numpy()
    t = timed(lambda: O.step(z4, np.float32(0.8), 0, 0), reps=1)
    out["c4_step_s"], out["c4_positions_per_s"] = t, L / t
    del z1, z2, z4
    # the full C2 run: the sharpening denoiser's logits for every step made
    # beforehand, so that the timed loop is the oracle's own
    steps_z = {}
    for s in range(48):
        steps_z[s] = synth.sharpening_logits(1002, s, L, V, m0_max=6.0, dtype=torch.bfloat16)
        if s >= 15:
            break
    n_used = [0]

    def den(s, canvas):
        n_used[0] = s + 1
        z = steps_z.get(s)
        if z is None:
            z = synth.sharpening_logits(1002, s, L, V, m0_max=6.0, dtype=torch.bfloat16)
        return z.to(torch.float64).numpy()

    t0 = time.perf_counter()
    _, n, stopped, _ = O.run(den, 0, L, V, n_sched=16)
    out["c2_run_s"], out["c2_run_steps"], out["c2_run_stopped"] = time.perf_counter() - t0, n, bool(stopped)
    out["c2_run_note"] = "includes widening each step's bf16 logits to fp64"
    del steps_z
    jobs = [((1003 << 32) | c, c, L, V) for c in range(16)]
    ctx = mp.get_context("spawn")
    with ctx.Pool(processes=workers) as pool:
        t0 = time.perf_counter()
        per = pool.map(_oracle_canvas_worker, jobs)
        wall = time.perf_counter() - t0
    used = min(workers, len(jobs))
    out["c3_step_workers"] = used
    out["c3_step_oracle_s_per_canvas"] = [round(x, 3) for x in per]
    out["c3_positions_per_s"] = len(jobs) * L / (sum(per) / used)
    out["c3_note"] = ("one canvas per task over the worker processes, each generating its own logits; "
                      "the rate divides the 16 canvases' positions by their summed oracle time over "
                      "the workers")
    out["c3_pool_wall_s"] = wall
    return out


def _time_graphs(graphs, k, torch):
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(k):
        graphs[i % len(graphs)].replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / 1e3


def read_ceiling_leg(torch, buffers, stream, k):
    """The rate of a plain streaming read (libdgprobe.so) over the same rotating
    logits buffers, for a few launch shapes; the best one is the measured
    ceiling that the statistics pass is set against."""
    from canvas_sampler_amd import probe

    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    nbytes = buffers[0].numel() * buffers[0].element_size()
    shapes = [(256, 512), (512, 256), (2048, 256), (4096, 1024), (8192, 1024)]
    best = None
    with torch.cuda.stream(stream):
        for grid, block in shapes:
            def launch(r, grid=grid, block=block):
                probe.stream_read(buffers[r], grid, block, sink, stream)
            for i in range(20):
                launch(i % len(buffers))
            start = torch.cuda.Event(enable_timing=True)
            stop = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            start.record()
            for i in range(k):
                launch(i % len(buffers))
            stop.record()
            torch.cuda.synchronize()
            us = start.elapsed_time(stop) * 1e3 / k
            if best is None or us < best[0]:
                best = (us, grid, block)
    us, grid, block = best
    return {"kernel": "stream_read_kernel", "avg_kernel_us": us, "GB/s": nbytes / us * 1e-3,
            "frac_of_peak": nbytes / us * 1e-3 / PEAK_HBM_GBS, "grid": grid, "block": block,
            "bytes_per_launch": nbytes, "shapes_tried": len(shapes)}


def sweep_leg(torch, B, synth):
    """Whole steps at other batch sizes (bf16, V = 262144) and the fp32
    single canvas: steps/s, positions/s and the statistics kernel's achieved
    HBM bandwidth (algorithmic bytes over its own time, HIP events)."""
    L, V = 256, 262144
    out = []
    for Bn, dtype, R, k in ((4, torch.bfloat16, 2, 200), (16, torch.bfloat16, 2, 60),
                            (64, torch.bfloat16, 2, 20), (1, torch.float32, 2, 400)):
        params = B.params_default(canvas_len=L, vocab=V)
        ctx = B.Context(params, max_batch=Bn)
        z = [torch.empty(Bn * L, V, dtype=dtype, device="cuda") for _ in range(R)]
        for r in range(R):
            for c in range(Bn):
                synth.sharpening_logits(1003 + c, r, L, V, m0_max=6.0, dtype=dtype, device="cuda",
                                        out=z[r][c * L:(c + 1) * L])
        temps = torch.full((Bn,), 0.6, device="cuda")
        seeds = torch.arange(Bn, dtype=torch.int64, device="cuda")
        canvas = torch.empty(Bn * L, dtype=torch.int32, device="cuda")
        ent = torch.empty(Bn * L, device="cuda")
        am = torch.empty(Bn * L, dtype=torch.int32, device="cuda")
        smp = torch.empty(Bn * L, dtype=torch.int32, device="cuda")
        o = ctx.step_out(canvas)
        stream = torch.cuda.Stream()
        # the inputs were made on the default stream: let that work finish (and
        # its freed temporaries stop being in use) before launching on `stream`
        torch.cuda.synchronize()

        def timed(fn):
            with torch.cuda.stream(stream):
                for i in range(3):
                    fn(i)
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                for i in range(k):
                    fn(i)
                e1.record()
                torch.cuda.synchronize()
            return e0.elapsed_time(e1) / 1e3 / k

        step_s = timed(lambda i: ctx.dg_sampler_step(z[i % R], temps, 1, seeds, o))
        stats_s = timed(lambda i: ctx.dg_canvas_stats(z[i % R], temps, 1, seeds, ent, am, smp))
        nbytes = Bn * L * V * z[0].element_size()
        out.append({"batch": Bn, "dtype": "bf16" if dtype == torch.bfloat16 else "f32",
                    "steps_per_s": 1.0 / step_s, "positions_per_s": Bn * L / step_s,
                    "stats_us": stats_s * 1e6, "stats_gbs": nbytes / stats_s / 1e9,
                    "stats_frac_of_8tbs": nbytes / stats_s / 1e9 / PEAK_HBM_GBS})
        ctx.close()
        del z
        torch.cuda.empty_cache()
    return out


def exp_b_leg(torch, B, synth):
    """The confidence-growth and entropy-bound sweeps of the pages' EXP B on
    the single-canvas workload (256 x 262144 bf16 sharpening logits, T 0.8 ->
    0.4 over 16 steps): steps to the adaptive stop and wall time of the whole
    loop (dg_run_canvas, logits made by the generator each step, one stop-flag
    read per step) for growth 0.75/1.5/3/6 per step, and commits per step for
    bounds 0.01/0.1/1/10."""
    L, V = 256, 262144
    torch.cuda.synchronize()
    out = {"growth": [], "bound": []}
    logits = torch.empty(L, V, dtype=torch.bfloat16, device="cuda")
    final = torch.empty(1, L, dtype=torch.int32, device="cuda")
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V, temp_steps=16), max_batch=1)
    for growth in (0.75, 1.5, 3.0, 6.0):
        def den(step, canvas_ptr, active_ptr, lg, stream, g=growth):
            synth.sharpening_logits(1002, step, L, V, m0_max=6.0, growth=g, dtype=torch.bfloat16,
                                    device="cuda", out=lg)
        ctx.dg_run_canvas([0], den, logits, final)       # warm-up
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        steps, stopped = ctx.dg_run_canvas([0], den, logits, final)
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        out["growth"].append({"growth": growth, "steps": int(steps[0]), "stopped": bool(stopped[0]),
                              "run_ms": 1e3 * dt, "ms_per_step": 1e3 * dt / max(1, steps[0])})
    ctx.close()
    for bound in (0.01, 0.1, 1.0, 10.0):
        ctx = B.Context(B.params_default(canvas_len=L, vocab=V, temp_steps=16, entropy_bound=bound),
                        max_batch=1)
        am = [torch.empty(L, dtype=torch.int32, device="cuda") for _ in range(2)]
        canvas = torch.empty(L, dtype=torch.int32, device="cuda")
        nacc = torch.empty(1, dtype=torch.int32, device="cuda")
        stop = torch.empty(1, dtype=torch.uint8, device="cuda")
        seeds = torch.zeros(1, dtype=torch.int64, device="cuda")
        counts = []
        for s in range(48):
            synth.sharpening_logits(1002, s, L, V, m0_max=6.0, dtype=torch.bfloat16, device="cuda",
                                    out=logits)
            temp = torch.tensor([B.dg_temperature(ctx.params, s)], device="cuda")
            o = ctx.step_out(canvas, argmax_out=am[s & 1], n_accept_out=nacc, stop_out=stop)
            ctx.dg_sampler_step(logits, temp, s, seeds, o, prev_argmax=am[(s + 1) & 1] if s else None)
            counts.append(int(nacc.item()))
            if stop.item():
                break
        out["bound"].append({"bound": bound, "steps": len(counts),
                             "commits_per_step": sum(counts) / len(counts)})
        ctx.close()
    return out


def run_loop_leg(torch, B, synth, reps=5):
    """The whole 48-step loop of one canvas at 256 x 262144 bf16, three ways:
    the host loop (dg_run_canvas: one stop-flag read and wait per step), the
    device-resident loop (dg_run_canvas_resident, stop flags kept on the
    device, no wait) and that loop captured once into a HIP graph and
    replayed. The denoiser does nothing and the logits are the sharpening
    denoiser's first step, which never meets the stop rule, so every run takes
    all 48 steps over the same 128 MiB logits buffer; what differs between the
    three is the loop's own overhead."""
    L, V, cap = 256, 262144, 48
    params = B.params_default(canvas_len=L, vocab=V, temp_steps=16, max_steps=cap)
    ctx = B.Context(params, max_batch=1)
    logits = synth.sharpening_logits(1002, 0, L, V, m0_max=6.0, dtype=torch.bfloat16, device="cuda")
    final = torch.empty(1, L, dtype=torch.int32, device="cuda")
    steps = torch.empty(1, dtype=torch.int32, device="cuda")
    stopped = torch.empty(1, dtype=torch.uint8, device="cuda")
    seeds = torch.zeros(1, dtype=torch.int64, device="cuda")
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def den(step, canvas_ptr, active_ptr, lg, strm):
        return None

    def wall(fn):
        fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / reps

    out = {}
    with torch.cuda.stream(stream):
        def host():
            st, sp = ctx.dg_run_canvas([0], den, logits, final)
            assert st == [cap] and sp == [False]
        out["host_loop_ms"] = 1e3 * wall(host)
        for k in (0, 8):
            out[f"resident_check{k}_ms"] = 1e3 * wall(
                lambda k=k: ctx.dg_run_canvas_resident(seeds, den, logits, final, steps, stopped,
                                                       check_every=k))
            assert steps.item() == cap and stopped.item() == 0
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            ctx.dg_run_canvas_resident(seeds, den, logits, final, steps, stopped, check_every=0)
        torch.cuda.synchronize()
        steps.fill_(-1)
        out["resident_graph_ms"] = 1e3 * wall(graph.replay)
        assert steps.item() == cap
    for k in list(out):
        out[k.replace("_ms", "_us_per_step")] = out[k] * 1e3 / cap
    out.update(workload="one canvas, 256 x 262144 bf16, 48 steps (no stop), no-op denoiser, "
                        "one logits buffer", steps=cap, reps=reps)
    ctx.close()
    return out


def generate_leg(torch, B, synth, n_canvases=4, reps=3):
    """Block-autoregressive generation of one stream of 4 canvases (1024
    tokens) at 256 x 262144 bf16 with the chained sharpening stand-in (canvas
    k sharpens on targets that continue canvas k-1; fresh N(0,1) logits each
    step, written by the stand-in on the device). Reports steps per canvas,
    tokens per forward (one cache-update forward per canvas counted), wall
    time, TPS = tokens / wall time, t_fwd = wall time / forwards, and the
    stand-in's own time per step, for the device loop checking its stop flags
    every step and every 4 steps."""
    L, V = 256, 262144
    params = B.params_default(canvas_len=L, vocab=V, temp_steps=16)
    ctx = B.Context(params, max_batch=1)
    logits = torch.empty(L, V, dtype=torch.bfloat16, device="cuda")
    tokens = torch.empty(1, n_canvases * L, dtype=torch.int32, device="cuda")
    steps = torch.empty(n_canvases, 1, dtype=torch.int32, device="cuda")
    stopped = torch.empty(n_canvases, 1, dtype=torch.uint8, device="cuda")
    seeds = torch.zeros(1, dtype=torch.int64, device="cuda")
    gen = 1002
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    state = {}

    def denoise(k, step, canvas_ptr, active_ptr, lg, strm):
        tgt, m0 = state[k]
        synth.chained_logits(gen, k, step, tgt, m0, V, dtype=torch.bfloat16, device="cuda", out=lg)

    def cache_update(k, canvas_ptr, strm):
        fin = torch.empty(L, dtype=torch.int32, device="cuda")
        B.copy_from_device(fin, canvas_ptr)
        state[k + 1] = synth.chained_targets(gen, k + 1, fin, L, V, device="cuda")

    out = {"workload": f"one stream of {n_canvases} canvases ({n_canvases * L} tokens), 256 x 262144 "
                       "bf16, chained sharpening stand-in (fresh N(0,1) logits per step on the "
                       "device), T 0.8->0.4 over 16 steps, b = 0.1", "canvases": n_canvases}
    with torch.cuda.stream(stream):
        for check_every in (1, 4):
            times = []
            for _ in range(reps + 1):
                state.clear()
                state[0] = synth.chained_targets(gen, 0, None, L, V, device="cuda")
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                ctx.dg_generate(seeds, n_canvases, denoise, cache_update, logits, tokens, steps,
                                stopped, check_every=check_every)
                torch.cuda.synchronize()
                times.append(time.perf_counter() - t0)
            wall = min(times[1:])
            st = steps.cpu().numpy()
            _, tpf = B.tokens_per_forward(st, L)
            fwd = int(st.sum()) + n_canvases
            out[f"check{check_every}"] = {"wall_ms": 1e3 * wall, "tps": n_canvases * L / wall,
                                          "t_fwd_us": 1e6 * wall / fwd}
        out["steps_per_canvas"] = st[:, 0].tolist()
        out["stopped"] = [bool(x) for x in stopped.cpu().numpy()[:, 0]]
        out["tpf"] = tpf
        out["forwards"] = fwd
        # the stand-in alone, to separate its share of t_fwd from the sampler's
        tgt, m0 = state[0]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(20):
            synth.chained_logits(gen, 0, i, tgt, m0, V, dtype=torch.bfloat16, device="cuda", out=logits)
        torch.cuda.synchronize()
        out["stand_in_us_per_step"] = 1e6 * (time.perf_counter() - t0) / 20
    ctx.close()
    return out


PEAK_FP32_MFMA_TFLOPS = 157.3


def selfcond_leg(torch, B, synth, k=200, d=30):
    """The sampling stage of the benchmark canvas with the self-conditioning
    matmul: statistics pass, then out = softmax(z/T) @ E with E fp32
    [262144, 30] (7.86 M parameters), over the same 4 rotating 128 MiB bf16
    logits buffers. Reports the matmul's time, its fp32 matrix-core rate
    (2 * rows * V * d flops) and the HBM rate of its logits and embedding
    reads, and the whole stage (statistics + self-conditioning)."""
    L, V, R = 256, 262144, 4
    params = B.params_default(canvas_len=L, vocab=V, temp_steps=16)
    ctx = B.Context(params, max_batch=1)
    logits = [synth.sharpening_logits(1002, r, L, V, m0_max=6.0, dtype=torch.bfloat16, device="cuda")
              for r in range(R)]
    E = synth.selfcond_embedding(5, V, d, device="cuda")
    temps = [torch.tensor([B.dg_temperature(params, r)], device="cuda") for r in range(R)]
    seeds = torch.zeros(1, dtype=torch.int64, device="cuda")
    ent = torch.empty(L, device="cuda")
    smp = torch.empty(L, dtype=torch.int32, device="cuda")
    am = [torch.empty(L, dtype=torch.int32, device="cuda") for _ in range(R)]
    out = torch.empty(L, d, device="cuda")
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()

    def stats(r):
        ctx.dg_canvas_stats(logits[r], temps[r], r, seeds, ent, am[r], smp)

    def sc(r):
        ctx.dg_self_condition(logits[r], temps[r], am[r], E, out)

    def stage(r):
        stats(r)
        sc(r)

    canvas = torch.empty(L, dtype=torch.int32, device="cuda")
    stop = torch.empty(1, dtype=torch.uint8, device="cuda")

    def step_sc(r):
        out = ctx.step_out(canvas, argmax_out=am[r], stop_out=stop)
        ctx.dg_sampler_step_selfcond(logits[r], temps[r], r, seeds, E, out_sc, out,
                                     prev_argmax=am[(r + 1) % R])

    out_sc = torch.empty(L, d, device="cuda")

    def timed(fn):
        for i in range(20):
            fn(i % R)
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(k):
            fn(i % R)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) * 1e3 / k

    with torch.cuda.stream(stream):
        for r in range(R):
            stats(r)
        t_sc = timed(sc)
        t_stage = timed(stage)
        t_step_sc = timed(step_sc)
    flops = 2.0 * L * V * d
    nbytes = L * V * 2 + V * d * 4
    ctx.close()
    return {"workload": "256 x 262144 bf16 logits (4 rotating buffers), E fp32 [262144, 30]",
            "kernel": "self_cond_kernel", "sc_us": t_sc, "tflops": flops / t_sc * 1e-6,
            "peak_fp32_mfma_tflops": PEAK_FP32_MFMA_TFLOPS,
            "mfma_frac": flops / t_sc * 1e-6 / PEAK_FP32_MFMA_TFLOPS,
            "read_gbs": nbytes / t_sc * 1e-3, "flops_per_launch": flops, "bytes_per_launch": nbytes,
            "stage_us": t_stage, "step_with_selfcond_us": t_step_sc,
            "step_with_selfcond_per_s": 1e6 / t_step_sc}


def lmhead_leg(args, torch, B, synth, keep=None):
    """The 64-canvas step whose logits come from the LM head: hidden bf16
    [16384, 2048] ~ N(0,1), weight bf16 [2048, 262144] ~ N(0, 1/2048), canvas c
    at step c mod 48 of the default schedule, seed c. Timed: the fused step
    (product with the statistics epilogue, merge of the tile partials,
    acceptance; the logits never stored) and, for comparison, the product
    alone with its 16 GiB of fp32 logits stored."""
    L, K, V, Bn = 256, 2048, 262144, 64
    params = B.params_default(canvas_len=L, vocab=V)
    ctx = B.Context(params, max_batch=Bn)
    hidden, weight = synth.lmhead_operands(1005, Bn * L, K, V, device="cuda")
    steps = torch.tensor([c % 48 for c in range(Bn)], dtype=torch.int32, device="cuda")
    temps = torch.tensor([B.dg_temperature(params, c % 48) for c in range(Bn)], device="cuda")
    seeds = torch.arange(Bn, dtype=torch.int64, device="cuda")
    canvas = torch.empty(Bn * L, dtype=torch.int32, device="cuda")
    out = ctx.step_out(canvas)
    ws = torch.empty(ctx.dg_lmhead_workspace_bytes(Bn), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    # the inputs were made on the default stream: let that work finish (and
    # its freed temporaries stop being in use) before launching on `stream`
    torch.cuda.synchronize()
    k = max(1, args.lmhead_steps)

    def timed(fn):
        with torch.cuda.stream(stream):
            fn()
            torch.cuda.synchronize()
            start = torch.cuda.Event(enable_timing=True)
            stop = torch.cuda.Event(enable_timing=True)
            start.record()
            for _ in range(k):
                fn()
            stop.record()
            torch.cuda.synchronize()
        return start.elapsed_time(stop) / 1e3 / k

    step_s = timed(lambda: ctx.dg_lmhead_sampler_step(hidden, weight, ws, temps, 0, seeds, out, steps=steps))
    gemm_s = None
    if not args.lmhead_no_store:
        logits = torch.empty(Bn * L, V, device="cuda")
        gemm_s = timed(lambda: ctx.dg_lmhead_logits(hidden, weight, logits))
        del logits
        torch.cuda.synchronize()
    flops = 2.0 * Bn * L * V * K
    tflops = flops / step_s / 1e12
    if keep is not None:
        # canvas 0 (step 0, T 0.8, seed 0) once more with every output, and its
        # rows of the product, for the oracle comparison of the CPU-baseline leg
        bufs = _step_buffers(torch, Bn, L)
        ctx.dg_lmhead_sampler_step(hidden, weight, ws, temps, 0, seeds, ctx.step_out(**bufs), steps=steps)
        z0 = torch.empty(L, V, device="cuda")
        ctx.dg_lmhead_logits(hidden[:L], weight, z0)
        torch.cuda.synchronize()
        keep.update(hidden=hidden[:L].to(torch.float32).cpu().numpy(),
                    weight=weight.to(torch.float32).cpu().numpy(), logits=z0.cpu().numpy(),
                    gpu=_host_outputs(bufs, 1, L)[0], temp=float(temps[0].item()), step=0, seed=0)
    ctx.close()
    rec = {"workload": "64 canvases x 256 positions, LM head bf16 [16384,2048] x [2048,262144] "
                       "with the statistics in the product's epilogue (logits never stored) -> "
                       "merge of the tile partials -> acceptance; per-canvas steps c mod 48",
           "fused_kernel": "lmhead_gemm_kernel<statistics epilogue>", "step_ms": step_s * 1e3,
           "step_tflops": tflops, "mfma_peak_tflops": PEAK_BF16_TFLOPS,
           "step_mfma_frac": tflops / PEAK_BF16_TFLOPS, "flops_per_launch": flops,
           "workspace_bytes": int(ws.numel()),
           "positions_per_s": Bn * L / step_s, "steps_per_s": 1.0 / step_s, "timed_launches": k}
    if gemm_s is not None:
        rec.update(store_gemm_ms=gemm_s * 1e3, store_gemm_tflops=flops / gemm_s / 1e12,
                   store_gemm_note="the same product alone, its 16 GiB of fp32 logits stored")
    return rec


def _step_buffers(torch, n, L):
    """Device buffers for every output of one step of n canvases."""
    dev = "cuda"
    return dict(canvas_out=torch.empty(n * L, dtype=torch.int32, device=dev),
                argmax_out=torch.empty(n * L, dtype=torch.int32, device=dev),
                sample_out=torch.empty(n * L, dtype=torch.int32, device=dev),
                accept_out=torch.empty(n * L, dtype=torch.uint8, device=dev),
                entropy_out=torch.empty(n * L, device=dev),
                n_accept_out=torch.empty(n, dtype=torch.int32, device=dev),
                mean_entropy_out=torch.empty(n, device=dev),
                stop_out=torch.empty(n, dtype=torch.uint8, device=dev))


def _host_outputs(bufs, n, L):
    """Per-canvas host dicts of one step's outputs."""
    g = {k: v.cpu().numpy() for k, v in bufs.items()}
    out = []
    for c in range(n):
        sl = slice(c * L, (c + 1) * L)
        out.append(dict(entropy=g["entropy_out"][sl], argmax=g["argmax_out"][sl], sample=g["sample_out"][sl],
                        accept=g["accept_out"][sl], n_accept=g["n_accept_out"][c], canvas=g["canvas_out"][sl],
                        mean_entropy=g["mean_entropy_out"][c], stop=g["stop_out"][c]))
    return out


def cpu_baseline_leg(torch, B, synth, c2, c5):
    """The oracle on the host cores, on bounded samples of each workload, and
    its agreement with the GPU on the very same inputs.

    Timing (cpu_baseline): the oracle as it stands (oracle.sampler's row
    statistics and decisions; oracle.parallel only spreads rows over a thread
    pool) on the benchmark's own four logits buffers (single canvas, 256 x
    262144 bf16, steps 0-3 of the 16-step schedule), all host threads up to 16;
    one of those steps is also timed on one thread.

    Agreement (parity): each sample's GPU outputs against the oracle's under
    the test suite's comparison policy (tests/full_parity.py compare_step:
    |dH| <= 1e-4, bit-exact integers except counted near-ties): C1 one step;
    C2 the four benchmark steps; C3 one step of 16 canvases (step 6, row
    loop); C4 two steps; C5 canvas 0 of the LM-head step (its oracle logits
    are the exact fp64 products)."""
    import numpy as np

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from full_parity import Tally, compare_step
    from oracle import parallel as OPAR

    L = 256
    threads = OPAR.default_threads()
    b32, thr32 = np.float32(0.1), np.float32(0.005)

    def host(t):
        return t.to("cpu").to(torch.float32).numpy()

    def job(zc, V, temp, seed, step, prev=None):
        return dict(rows=lambda r0, r1, zc=zc: zc[r0:r1], L=L, V=V, temp=np.float32(temp), seed=seed,
                    step=step, prev_argmax=prev)

    def compare(tally, gpu, orc, label, **kw):
        try:
            compare_step(gpu, orc, label, tally, b32, thr32, **kw)
        except AssertionError as e:
            tally.clauses.append(f"MISMATCH {e}")

    def gpu_step(V, zs, temps, seeds, step, dtype, prev=None):
        n = len(seeds)
        ctx = B.Context(B.params_default(canvas_len=L, vocab=V), max_batch=n)
        z = torch.cat(zs) if len(zs) > 1 else zs[0]
        bufs = _step_buffers(torch, n, L)
        ctx.dg_sampler_step(z, torch.tensor(temps, device="cuda"), step,
                            torch.tensor(seeds, dtype=torch.int64, device="cuda"), ctx.step_out(**bufs),
                            prev_argmax=prev)
        torch.cuda.synchronize()
        out = _host_outputs(bufs, n, L)
        ctx.close()
        return out

    parity = {}
    # C2: the benchmark's buffers; steps r = 0..3 chained by the previous argmax
    tally = Tally("C2")
    jobs, prev = [], None
    for r in range(len(c2["logits"])):
        jobs.append(job(host(c2["logits"][r]), 262144, c2["temps"][r], 0, r, prev))
        prev = c2["gpu"][r]["argmax"].astype(np.int64)
    # the four steps over the thread pool, repeated for about 8 s of wall time
    reps, t0 = 0, time.perf_counter()
    while reps == 0 or time.perf_counter() - t0 < 8.0:
        orcs = OPAR.steps(jobs, threads=threads, bound=b32, stop_threshold=thr32)
        reps += 1
    t_all = time.perf_counter() - t0
    t0 = time.perf_counter()
    OPAR.steps(jobs[:1], threads=1, bound=b32, stop_threshold=thr32)
    t_one = time.perf_counter() - t0
    for r, (g, o) in enumerate(zip(c2["gpu"], orcs)):
        compare(tally, g, o, f"C2 step {r}")
    parity["C2"] = tally.record()
    cpu = {"value": reps * len(jobs) / t_all, "unit": "steps/s", "cores": threads, "kind": "oracle",
           "sample": f"{reps} x {len(jobs)} full oracle steps of the benchmark workload (its 4 logits buffers: "
                     f"256 rows x 262144 bf16, steps 0-3), fp64 numpy row statistics over {threads} "
                     f"threads ({os.cpu_count()} host CPUs visible)",
           "single_thread_steps_per_s": 1.0 / t_one, "seconds": t_all + t_one}
    del jobs, orcs

    # C1: one margin step, 256 x 4096 fp32
    tally = Tally("C1")
    z = synth.margin_logits(1001, L, 4096, m_max=12.0, dtype=torch.float32, device="cuda")
    g = gpu_step(4096, [z], [0.8], [0], 0, torch.float32)[0]
    compare(tally, g, OPAR.steps([job(host(z), 4096, 0.8, 0, 0)], threads=threads)[0], "C1")
    parity["C1"] = tally.record()

    # C3: one step of 16 canvases (step 6 of the 16-step schedule)
    tally = Tally("C3")
    n, step = 16, 6
    t = B.dg_temperature(B.params_default(temp_steps=16), step)
    zs = [synth.sharpening_logits((1003 << 32) | c, step, L, 262144, m0_max=8.0, dtype=torch.bfloat16,
                                  device="cuda") for c in range(n)]
    gs = gpu_step(262144, zs, [t] * n, list(range(n)), step, torch.bfloat16)
    orcs = OPAR.steps([job(host(zs[c]), 262144, t, c, step) for c in range(n)], threads=threads)
    for c in range(n):
        compare(tally, gs[c], orcs[c], f"C3 canvas {c}")
    parity["C3"] = tally.record()
    del zs, orcs

    # C4: steps 0 and 1 of the untrained stand-in (fp32 iid N(0, 0.05))
    tally = Tally("C4")
    prev_g, prev_o = None, None
    params = B.params_default()
    for step in range(2):
        z = synth.iid_normal_logits(1004, step, L, 262144, variance=0.05, dtype=torch.float32, device="cuda")
        t = B.dg_temperature(params, step)
        g = gpu_step(262144, [z], [t], [0], step, torch.float32, prev=prev_g)[0]
        o = OPAR.steps([job(host(z), 262144, t, 0, step, prev_o)], threads=threads)[0]
        compare(tally, g, o, f"C4 step {step}")
        prev_g = torch.as_tensor(g["argmax"], device="cuda")
        prev_o = o["argmax"]
    parity["C4"] = tally.record()

    # C5: canvas 0 of the fused LM-head step; the oracle runs on the product's
    # own fp32 logits (the fused kernel's input bit for bit), whose distance
    # from the exact fp64 products is reported beside it
    if c5:
        tally = Tally("C5")
        from oracle import lmhead as OL
        exact = OL.logits(c5["hidden"], c5["weight"])
        z0 = c5["logits"].astype(np.float64)
        err = np.abs(z0 - exact).max(axis=1)
        del exact
        o = OPAR.steps([job(z0, z0.shape[1], c5["temp"], c5["seed"], c5["step"])], threads=threads)[0]
        compare(tally, c5["gpu"], o, "C5 canvas 0")
        parity["C5"] = dict(tally.record(), max_logit_error=float(err.max()),
                            note="canvas 0 of 64 (step 0, T 0.8); oracle on the product's fp32 logits, "
                                 "max_logit_error against the exact fp64 products")
    for rec in parity.values():
        rec["match"] = not any(c.startswith("MISMATCH") for c in rec["clauses"])
    return cpu, parity


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--rotate", type=int, default=4, help="logits buffers (>= 4 beats the LLC)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-lmhead", action="store_true", help="skip the LM-head step")
    ap.add_argument("--no-sweep", action="store_true", help="skip the batch and dtype sweep")
    ap.add_argument("--no-exp-b", action="store_true", help="skip the confidence-growth and bound sweeps")
    ap.add_argument("--no-selfcond", action="store_true",
                    help="skip the self-conditioning matmul of the sampling stage")
    ap.add_argument("--no-generate", action="store_true",
                    help="skip the block-autoregressive generation of four canvases (TPF/TPS)")
    ap.add_argument("--no-run-loop", action="store_true",
                    help="skip the host-loop / device-resident / graph comparison of the 48-step loop")
    ap.add_argument("--lmhead-only", action="store_true",
                    help="only run the LM-head product and step (for counter runs)")
    ap.add_argument("--lmhead-steps", type=int, default=10)
    ap.add_argument("--lmhead-no-store", action="store_true",
                    help="skip timing the product alone with its logits stored")
    ap.add_argument("--cpu-full", action="store_true",
                    help="only time the oracle on the host for C1-C4 single steps, the full C2 run "
                         "and C3 over processes (a few minutes; no GPU work)")
    ap.add_argument("--cpu-workers", type=int, default=16)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 20 plain 128 MiB device copies (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the sampler has no multi-GPU path (independent "
              "canvases would shard across GPUs without any communication)", file=sys.stderr)
        sys.exit(2)

    if args.cpu_full:
        print(json.dumps({"cpu_oracle": cpu_full_leg(max(1, args.cpu_workers)),
                          "host_cpus": os.cpu_count()}), flush=True)
        return

    import numpy as np
    import torch

    from canvas_sampler_amd import binding as B
    from canvas_sampler_amd import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        src = torch.ones(64 << 20, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copy", "bytes_read": src.numel() * 2,
                          "bytes_written": dst.numel() * 2, "launches": 20}))
        return
    if args.lmhead_only:
        print(json.dumps({"lmhead": lmhead_leg(args, torch, B, synth)}), flush=True)
        return
    L, V, Bn = 256, 262144, 1
    R = max(1, args.rotate)
    params = B.params_default(canvas_len=L, vocab=V, temp_steps=16)
    ctx = B.Context(params, max_batch=Bn)
    dev = "cuda"
    logits = [synth.sharpening_logits(1002, r, L, V, m0_max=6.0, dtype=torch.bfloat16, device=dev)
              for r in range(R)]
    temps = [torch.tensor([B.dg_temperature(params, r)], device=dev) for r in range(R)]
    seeds = torch.tensor([0], dtype=torch.int64, device=dev)
    am = [torch.empty(L, dtype=torch.int32, device=dev) for _ in range(2)]
    canvas = torch.empty(L, dtype=torch.int32, device=dev)
    stop = torch.empty(1, dtype=torch.uint8, device=dev)
    nacc = torch.empty(1, dtype=torch.int32, device=dev)
    ent = torch.empty(L, device=dev)
    smp = torch.empty(L, dtype=torch.int32, device=dev)
    stream = torch.cuda.Stream()
    # the inputs were made on the default stream: let that work finish (and
    # its freed temporaries stop being in use) before launching on `stream`
    torch.cuda.synchronize()

    def full_step(r):
        out = ctx.step_out(canvas, argmax_out=am[r & 1], stop_out=stop, n_accept_out=nacc)
        ctx.dg_sampler_step(logits[r], temps[r], r, seeds, out, prev_argmax=am[(r + 1) & 1])

    def stats_only(r):
        ctx.dg_canvas_stats(logits[r], temps[r], r, seeds, ent, am[r & 1], smp)

    def capture(fn):
        graphs = []
        with torch.cuda.stream(stream):
            for r in range(R):
                fn(r)                      # eager warm-up outside capture
            torch.cuda.synchronize()
            for r in range(R):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    fn(r)
                graphs.append(g)
        torch.cuda.synchronize()
        return graphs

    step_graphs = capture(full_step)
    # one graph holding a step on each of the R buffers, so that the graph
    # launch is paid once per R steps
    multi_graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        with torch.cuda.graph(multi_graph, stream=stream):
            for r in range(R):
                full_step(r)
    torch.cuda.synchronize()

    def time_eager(fn, k):
        """HIP events on the launch stream around k back-to-back launches."""
        start = torch.cuda.Event(enable_timing=True)
        stop = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(k):
            fn(i % R)
        stop.record()
        torch.cuda.synchronize()
        return start.elapsed_time(stop) / 1e3

    with torch.cuda.stream(stream):
        time_eager(full_step, args.warmup)
        t_step = time_eager(full_step, args.steps)
        time_eager(stats_only, args.warmup)
        t_stats = time_eager(stats_only, args.steps)
        # the same steps replayed from captured HIP graphs, for reference
        _time_graphs(step_graphs, args.warmup, torch)
        t_graph = _time_graphs(step_graphs, args.steps, torch)
        n_multi = max(1, args.steps // R)
        _time_graphs([multi_graph], max(1, args.warmup // R), torch)
        t_graph_multi = _time_graphs([multi_graph], n_multi, torch)

    read_ceiling = read_ceiling_leg(torch, logits, stream, args.steps)
    steps_per_s = args.steps / t_step
    bytes_per_launch = Bn * L * V * 2
    stats_s = t_stats / args.steps
    achieved = bytes_per_launch / stats_s / 1e9
    traffic = _traffic(bytes_per_launch)

    # every output of one step on each benchmark buffer (steps 0..R-1, each
    # after the previous one), for the oracle comparison
    c2 = None
    if not args.no_cpu_baseline:
        c2 = {"logits": logits, "temps": [float(t.item()) for t in temps], "gpu": []}
        prev = None
        for r in range(R):
            bufs = _step_buffers(torch, 1, L)
            ctx.dg_sampler_step(logits[r], temps[r], r, seeds, ctx.step_out(**bufs), prev_argmax=prev)
            torch.cuda.synchronize()
            c2["gpu"].append(_host_outputs(bufs, 1, L)[0])
            prev = bufs["argmax_out"]

    rec = {
        "metric": METRIC, "value": steps_per_s, "unit": "steps/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": 1e3 * t_step / args.steps,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "single canvas, 256 positions x 262144 vocab, bf16 sharpening "
                               f"logits, {R} rotating 128 MiB buffers",
                   "batch": Bn, "canvas_len": L, "vocab": V, "entropy_bound": 0.1,
                   "temperature": "0.8->0.4 over 16 steps"},
        "positions_per_s": steps_per_s * Bn * L,
        "graph_steps_per_s": args.steps / t_graph,
        "graph_multi_steps_per_s": n_multi * R / t_graph_multi,
        "graph_multi_steps_per_graph": R,
        "roofline": {"bound": "hbm", "kernel": "canvas_stats_kernel", "achieved": achieved,
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": traffic, "avg_kernel_us": stats_s * 1e6,
                     "algorithmic_bytes_per_launch": bytes_per_launch,
                     "frac_of_read_ceiling": read_ceiling["GB/s"] and achieved / read_ceiling["GB/s"]},
        "read_ceiling": read_ceiling,
        "cpu_baseline": None,
        "parity": None,
        "sweep": None if args.no_sweep else sweep_leg(torch, B, synth),
        "exp_b": None if args.no_exp_b else exp_b_leg(torch, B, synth),
        "run_loop": None if args.no_run_loop else run_loop_leg(torch, B, synth),
        "generate": None if args.no_generate else generate_leg(torch, B, synth),
        "selfcond": None if args.no_selfcond else selfcond_leg(torch, B, synth),
    }
    c5 = {} if not args.no_cpu_baseline and not args.no_lmhead else None
    rec["lmhead"] = None if args.no_lmhead else lmhead_leg(args, torch, B, synth, keep=c5)
    if c2 is not None:
        rec["cpu_baseline"], rec["parity"] = cpu_baseline_leg(torch, B, synth, c2, c5)
    print(json.dumps(rec), flush=True)
    ctx.close()


if __name__ == "__main__":
    main()
