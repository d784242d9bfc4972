"""GPU tests of the block-autoregressive driver (dg_generate) against the
oracle's driver (oracle/blockar.py): per-canvas seeds, chaining through the
cache update, the tokens of every stream, steps and stop flags, and the TPF
accounting."""
import numpy as np
import pytest
import torch

from canvas_sampler_amd import binding as B
from canvas_sampler_amd import synth
from oracle import blockar as BA
from oracle import sampler as O

from gpu_util import gpu, require_gpu, seeds_tensor
from full_parity import trajectory

pytestmark = gpu


class ChainedDenoiser:
    """Device-side stand-in: canvas k of stream c sharpens on targets that
    continue stream c's canvas k-1 (synth.chained_targets / chained_logits).
    Records the canvas handed to every step and the state of every canvas."""

    def __init__(self, gens, L, V, dtype=torch.bfloat16, certain=False):
        self.gens, self.L, self.V, self.dtype, self.certain = gens, L, V, dtype, certain
        self.state = {0: [synth.chained_targets(g, 0, None, L, V, device="cuda") for g in gens]}
        self.canvas_in = {}
        self.finished = {}

    def denoise(self, k, step, canvas_ptr, active_ptr, logits, stream):
        Bn, L = len(self.gens), self.L
        buf = torch.empty(Bn, L, dtype=torch.int32, device="cuda")
        B.copy_from_device(buf, canvas_ptr)
        self.canvas_in[(k, step)] = buf
        for c, g in enumerate(self.gens):
            tgt, m0 = self.state[k][c]
            rows = logits[c * L:(c + 1) * L]
            if self.certain:
                rows.zero_()
                rows[torch.arange(L, device="cuda"), tgt] = 1000.0
            else:
                synth.chained_logits(g, k, step, tgt, m0, self.V, dtype=self.dtype, device="cuda",
                                     out=rows)

    def cache_update(self, k, canvas_ptr, stream):
        fin = torch.empty(len(self.gens), self.L, dtype=torch.int32, device="cuda")
        B.copy_from_device(fin, canvas_ptr)
        self.finished[k] = fin
        self.state[k + 1] = [synth.chained_targets(g, k + 1, fin[c], self.L, self.V, device="cuda")
                             for c, g in enumerate(self.gens)]


def _generate(ctx, seeds, n, den, dtype, check_every):
    Bn, L, V = len(seeds), ctx.L, ctx.V
    logits = torch.empty(Bn * L, V, dtype=dtype, device="cuda")
    tokens = torch.full((Bn, n * L), -1, dtype=torch.int32, device="cuda")
    steps = torch.full((n, Bn), -1, dtype=torch.int32, device="cuda")
    stopped = torch.full((n, Bn), 7, dtype=torch.uint8, device="cuda")
    ctx.dg_generate(seeds_tensor(seeds), n, den.denoise, den.cache_update, logits, tokens, steps,
                    stopped, check_every=check_every)
    torch.cuda.synchronize()
    return tokens.cpu().numpy(), steps.cpu().numpy(), stopped.cpu().numpy().astype(bool)


def test_canvas_seeds_match_oracle():
    # the device's per-canvas seeds, seen through the initial canvases: a
    # one-step run of canvas k starts from init_canvas(canvas_seed(seed, k))
    L, V, n = 64, 4096, 5
    seeds = [0, 2**63 + 5, 12345]
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V, max_steps=1), max_batch=3)
    den = ChainedDenoiser([1, 2, 3], L, V, dtype=torch.float32)
    _generate(ctx, seeds, n, den, torch.float32, 0)
    for k in range(n):
        got = den.canvas_in[(k, 0)].cpu().numpy()
        for c, s in enumerate(seeds):
            assert np.array_equal(got[c], O.init_canvas(BA.canvas_seed(s, k), L, V)), (k, c)


def test_certain_chain_closed_form():
    # one-hot logits at the chained targets: every canvas stops at its second
    # step with its targets as output, so TPF = n*L / (2n + n) exactly and the
    # tokens equal the brute-force chain of targets
    L, V, n = 256, 4096, 4
    gens, seeds = [5, 6], [0, 7]
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V, temp_steps=16), max_batch=2)
    for check_every in (0, 3):
        den = ChainedDenoiser(gens, L, V, dtype=torch.float32, certain=True)
        tokens, steps, stopped = _generate(ctx, seeds, n, den, torch.float32, check_every)
        assert (steps == 2).all() and stopped.all()
        for c, g in enumerate(gens):
            chain = [synth.chained_targets(g, 0, None, L, V, device="cuda")[0]]
            for k in range(1, n):
                chain.append(synth.chained_targets(g, k, chain[-1], L, V, device="cuda")[0])
            assert np.array_equal(tokens[c], torch.cat(chain).cpu().numpy())
        per, total = B.tokens_per_forward(steps, L)
        assert per == [n * L / (3 * n)] * 2 and total == n * L / (3 * n)


def test_generate_matches_oracle():
    # two streams of three canvases on the chained sharpening stand-in
    # (bf16, V = 4096): each canvas is run by the oracle from the same logits
    # bits (conditioned on the GPU's previous canvas, so that a difference
    # cannot carry over) and must stop where the oracle does with the same
    # argmax canvas, per-step differences only at counted near-ties; the
    # device loop's own variants (never waiting, waiting every 4 steps) agree
    # bit for bit
    L, V, n = 256, 4096, 3
    gens, seeds = [1002, 2002], [0, 2**63 + 5]
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V, temp_steps=16), max_batch=2)
    den = ChainedDenoiser(gens, L, V)
    tokens, steps, stopped = _generate(ctx, seeds, n, den, torch.bfloat16, 0)
    den4 = ChainedDenoiser(gens, L, V)
    t4, s4, st4 = _generate(ctx, seeds, n, den4, torch.bfloat16, 4)
    assert np.array_equal(t4, tokens) and np.array_equal(s4, steps) and np.array_equal(st4, stopped)
    for k in range(n):
        for c in range(2):
            assert np.array_equal(tokens[c, k * L:(k + 1) * L], den.finished[k][c].cpu().numpy())

        # canvas k of both streams, conditioned on the GPU's finished canvas
        # k - 1 (so that a difference cannot carry over), every row of every
        # step against the oracle
        def write(step, out, k=k):
            for c, g in enumerate(gens):
                tgt, m0 = den.state[k][c]
                synth.chained_logits(g, k, step, tgt, m0, V, dtype=torch.bfloat16, device="cuda",
                                     out=out[c * L:(c + 1) * L])

        tally, runs, _ = trajectory(f"generate canvas {k}", L, V, [BA.canvas_seed(sd, k) for sd in seeds],
                                    write, torch.bfloat16, temp_steps=16, library_loop=False)
        for c in range(2):
            assert (int(steps[k, c]), bool(stopped[k, c])) == runs[c][:2], f"stream {c} canvas {k}"
            assert np.array_equal(tokens[c, k * L:(k + 1) * L], runs[c][2]), f"stream {c} canvas {k}"
        tally.report()
    per, total = B.tokens_per_forward(steps, L)
    for c in range(2):
        assert per[c] == pytest.approx(BA.tokens_per_forward(steps[:, c].tolist(), L), rel=1e-15)
    print("steps", steps.tolist(), "TPF", per, total)


def test_argument_errors_and_callback_failures():
    L, V = 32, 4096
    require_gpu()
    ctx = B.Context(B.params_default(canvas_len=L, vocab=V, max_steps=6), max_batch=2)
    logits = torch.zeros(2 * L, V, device="cuda")
    tokens = torch.zeros(2, 3 * L, dtype=torch.int32, device="cuda")
    steps = torch.zeros(3, 2, dtype=torch.int32, device="cuda")
    stopped = torch.zeros(3, 2, dtype=torch.uint8, device="cuda")
    seeds = seeds_tensor([1, 2])
    noop = lambda *a: None
    with pytest.raises(B.DgError, match="n_canvases"):
        ctx.dg_generate(seeds, 0, noop, None, logits, tokens, steps, stopped)
    with pytest.raises(B.DgError, match="check_every"):
        ctx.dg_generate(seeds, 3, noop, None, logits, tokens, steps, stopped, check_every=-1)
    with pytest.raises(B.DgError, match="tokens is NULL"):
        ctx.dg_generate(seeds, 3, noop, None, logits, None, steps, stopped)
    final = torch.zeros(2, L, dtype=torch.int32, device="cuda")
    with pytest.raises(B.DgError, match="check_every"):
        ctx.dg_run_canvas_resident(seeds, noop, logits, final, steps[0], stopped[0], check_every=-2)

    class Boom(RuntimeError):
        pass

    def bad_cache(k, canvas_ptr, stream):
        if k == 1:
            raise Boom("cache update failed")

    with pytest.raises(Boom):
        ctx.dg_generate(seeds, 3, noop, bad_cache, logits, tokens, steps, stopped, check_every=2)
    torch.cuda.synchronize()
    # canvas 0 and 1 ran (zero logits never stop: the 6-step cap), canvas 2 did not start
    assert steps.cpu().numpy()[:2].tolist() == [[6, 6], [6, 6]]

    def bad_denoise(k, step, canvas_ptr, active_ptr, lg, stream):
        if k == 1 and step == 2:
            raise Boom("denoiser failed")

    with pytest.raises(Boom):
        ctx.dg_generate(seeds, 3, bad_denoise, None, logits, tokens, steps, stopped)
    torch.cuda.synchronize()
    # the context stays usable
    ctx.dg_generate(seeds, 3, noop, None, logits, tokens, steps, stopped, check_every=3)
    assert (steps.cpu().numpy() == 6).all() and not stopped.cpu().numpy().any()
    per, total = B.tokens_per_forward(steps.cpu().numpy(), L)
    assert total == 3 * L / (3 * 6 + 3)
