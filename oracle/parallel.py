"""Thread-parallel driver of the oracle over rows and canvases (test
infrastructure only: tests/, __graft_entry__.smoke() and bench.py's CPU
baseline leg call it; the product path never does).

It computes nothing of its own: sampler.row_statistics runs on chunks of rows
in a thread pool (numpy releases the interpreter lock inside its array
operations, so the chunks proceed in parallel), and sampler.decide runs once
per canvas on the gathered rows, exactly as sampler.step composes the two.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import sampler as S

# Rows per task: large enough that numpy's per-call overhead is negligible,
# small enough that a chunk's fp64 temporaries stay near 100 MB at V = 262144.
ROWS_PER_TASK = 16


def default_threads():
    """Threads for the pool: the host's CPUs, at most 16."""
    return max(1, min(16, os.cpu_count() or 1))


def steps(jobs, threads=None, bound=np.float32(0.1), stop_threshold=np.float32(0.005)):
    """One oracle step for each job, all jobs' rows sharing one thread pool.

    A job is a dict with
      rows(r0, r1)  -> logits of canvas rows r0..r1-1, [r1 - r0, V] (any
                       float dtype; widened exactly to fp64)
      L, V, temp, seed, step, prev_argmax (None at the first step).
    Returns one dict per job, with sampler.step's keys plus the sample's
    winning scores and margins (block_best, block_gap, elem_best, elem_gap)
    and the renoise tokens."""
    threads = threads or default_threads()
    tasks = [(i, r0) for i, j in enumerate(jobs) for r0 in range(0, j["L"], ROWS_PER_TASK)]

    def run(task):
        i, r0 = task
        j = jobs[i]
        r1 = min(r0 + ROWS_PER_TASK, j["L"])
        return S.row_statistics(j["rows"](r0, r1), j["temp"], j["seed"], np.arange(r0, r1), j["step"])

    with ThreadPoolExecutor(max_workers=threads) as pool:
        parts = list(pool.map(run, tasks))
    out, at = [], 0
    for j in jobs:
        n = -(-j["L"] // ROWS_PER_TASK)
        mine = parts[at:at + n]
        at += n
        rec = {k: np.concatenate([p[k] for p in mine]) for k in mine[0]}
        rec.update(S.decide(rec["entropy"], rec["argmax"], rec["sample"], j["seed"], j["step"], j["V"],
                            j["prev_argmax"], bound, stop_threshold))
        out.append(rec)
    return out
