"""LM-head projection of the fused configuration: logits = hidden . weight,
then one sampler step on those logits. Test infrastructure only (see the
package header).

The sampling stage of a denoising step runs a full-vocabulary softmax over the
256 canvas positions ("DiffusionGemma: Parallel Denoising From an
Autoregressive Checkpoint", the hardware breakdown of one step); its logits are
the decoder's last hidden states times the LM-head weights. This module writes
that product out plainly and hands the result to sampler.step.

Exactness: hidden and weight hold bf16 values (8 significant bits), so every
product h_k * w_k is exact in fp64, and the fp64 sum of K of them differs from
the real sum by at most about K * 2^-53 times the sum of their magnitudes
(below 1e-11 at K = 2048 with unit-scale logits). These logits stand for the
real-number product.
"""
import numpy as np

from . import sampler


def logits(hidden, weight, col_chunk=16384):
    """Exact-enough logits [rows, V] = hidden [rows, K] . weight [K, V] in fp64.

    hidden and weight may be any float arrays whose values are exactly
    representable in fp64 (bf16 or fp32 values widen exactly). The product is
    taken a block of vocabulary columns at a time only to bound memory."""
    h = np.asarray(hidden, dtype=np.float64)
    w = np.asarray(weight)
    rows, k = h.shape
    k2, vocab = w.shape
    if k != k2:
        raise ValueError(f"hidden has K = {k} but weight has {k2} rows")
    out = np.empty((rows, vocab), dtype=np.float64)
    for c0 in range(0, vocab, col_chunk):
        c1 = min(vocab, c0 + col_chunk)
        out[:, c0:c1] = h @ w[:, c0:c1].astype(np.float64)
    return out


def step(hidden, weight, temp, seed, step_index, prev_argmax=None,
         bound=np.float32(0.1), stop_threshold=np.float32(0.005)):
    """One sampler step of one canvas whose logits are hidden . weight.
    hidden: [L, K]; weight: [K, V]. Returns sampler.step's dict plus 'logits'."""
    z = logits(hidden, weight)
    out = sampler.step(z, temp, seed, step_index, prev_argmax=prev_argmax, bound=bound,
                       stop_threshold=stop_threshold)
    out["logits"] = z
    return out
