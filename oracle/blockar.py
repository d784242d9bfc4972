"""Block-autoregressive multi-canvas generation and its tokens-per-forward
accounting — the oracle (test infrastructure only).

What the pages say:
  "DiffusionGemma Lab" (shadowgraph.io), §2, Figure 1: the decoder denoises
  one 256-token canvas at a time and finished canvases chain
  block-autoregressively.
  "DiffusionGemma: When the LLM Stops Writing Left to Right" (LunarOps),
  "What DiffusionGemma Actually Is": block-autoregressive multi-canvas
  sampling generates one canvas at a time, each conditioned on the finished
  canvases before it; diffusion inside a canvas, autoregression across them.
  "DiffusionGemma: Parallel Denoising From an Autoregressive Checkpoint"
  (boxwrench.dev), "Finding": committed canvases are appended to the
  encoder's KV cache canvas by canvas, without re-encoding; tokens per
  forward pass (TPF) counts the extra forward pass that updates the cache,
  and throughput is TPS = TPF / t_fwd.

Readings where the pages are silent:
  - canvas k of a stream whose seed is s draws its random numbers with seed
    s_k: s_0 = s, and for k >= 1 s_k = w0 + 2^32 * w1 of the Philox4x32-10
    words for counter (k, 0, 0, CANVAS) under key(s);
  - the conditioning reaches canvas k only through the denoiser, which is
    told each finished canvas once (the cache update) before canvas k + 1;
  - every finished canvas costs one cache-update forward, the last one
    included; the prompt's own encoding is not counted;
  - a canvas is committed whole: every canvas contributes its L tokens, so
    TPF = (canvases * L) / (denoising steps + canvases).

Pinned in tests/test_oracle_blockar.py by closed forms (a never-confident
denoiser runs every canvas to the cap; a certain one stops every canvas at
its second step), by a brute-force chain of the certain denoiser's targets,
and by the Philox known-answer vectors behind the seed derivation. Shares no
code with the HIP implementation.
"""
import numpy as np

from .philox import TAG_CANVAS, philox4x32_10, seed_key
from .sampler import run


def canvas_seed(seed, k):
    """Seed of canvas k of the stream whose seed is `seed` (uint64 int)."""
    s = int(seed) & 0xFFFFFFFFFFFFFFFF
    if k == 0:
        return s
    k0, k1 = seed_key(s)
    w = philox4x32_10(k, 0, 0, TAG_CANVAS, k0, k1)
    return int(w[0]) | (int(w[1]) << 32)


def generate(denoise, cache_update, seed, n_canvases, canvas_len, vocab, **run_kw):
    """n_canvases canvases of one stream, one after the other.

    denoise(k, step, canvas) -> logits [L, V] of canvas k at `step`;
    cache_update(k, tokens) is told canvas k's final argmax canvas before
    canvas k + 1 starts (it may be None). Other keywords go to sampler.run.
    Returns (tokens [n_canvases * L], steps per canvas, stopped per canvas)."""
    tokens, steps, stopped = [], [], []
    for k in range(n_canvases):
        final, n, st, _ = run(lambda s, canvas, k=k: denoise(k, s, canvas), canvas_seed(seed, k),
                              canvas_len, vocab, **run_kw)
        if cache_update is not None:
            cache_update(k, final)
        tokens.append(np.asarray(final, dtype=np.int64))
        steps.append(int(n))
        stopped.append(bool(st))
    return np.concatenate(tokens), steps, stopped


def forwards(steps):
    """Forward passes of a stream: its denoising steps plus one cache update
    per canvas."""
    return int(sum(steps)) + len(steps)


def tokens_per_forward(steps, canvas_len):
    """TPF of a stream whose canvases took `steps` denoising steps each."""
    return len(steps) * canvas_len / forwards(steps)


def tokens_per_second(tpf, t_fwd):
    """TPS = TPF / t_fwd, t_fwd the time of one forward pass in seconds."""
    return tpf / t_fwd
