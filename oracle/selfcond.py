"""The self-conditioning matmul of the sampling stage — the oracle (test
infrastructure only).

What the pages say: "DiffusionGemma: Parallel Denoising From an
Autoregressive Checkpoint" (boxwrench.dev), "Finding": a self-conditioning
feedforward block of 7.8 million parameters feeds the previous step's
prediction back into the decoder and behaves like a token bottleneck; in the
hardware paragraph, the sampling stage of a denoising step runs the
full-vocabulary softmax together with the self-conditioning matmul, in full
precision, over the 256 canvas positions.

Reading (the pages give no shapes): the matmul is the expectation of a token
embedding under the step's prediction,
    s_r = sum_v p_r(v) * E[v, :],   p_r = softmax(z_r / T),
with E a [V, d] matrix holding the block's parameters (V * d = 7,864,320 at
V = 262144 and d = 30, i.e. 7.8 M); the prediction is the tempered softmax
the sampler computes in the same stage. The rest of the block (mapping s into
the decoder's width) belongs to the model and is not part of the sampler.

Plain fp64: softmax with the row maximum subtracted, then a library matmul.
Pinned in tests/test_oracle_selfcond.py by one-hot and uniform rows, a column
of ones (probabilities sum to one), set-indicator columns against brute-force
sums of probabilities, and the closed-form mean of a truncated geometric
distribution. Shares no code with the HIP implementation.
"""
import numpy as np


def softmax(z, temp):
    """Tempered softmax of each row of z in fp64."""
    x = np.asarray(z, dtype=np.float64) / np.float64(temp)
    x = x - x.max(axis=-1, keepdims=True)
    e = np.exp(x)
    return e / e.sum(axis=-1, keepdims=True)


def self_condition(z, temp, embed):
    """s [rows, d] = softmax(z / temp) @ embed, z [rows, V], embed [V, d]."""
    return softmax(z, temp) @ np.asarray(embed, dtype=np.float64)


def magnitude(z, temp, embed):
    """sum_v p_r(v) |E[v, n]| per row and column: the scale of each output's
    terms, against which a floating-point result's error is measured."""
    return softmax(z, temp) @ np.abs(np.asarray(embed, dtype=np.float64))
