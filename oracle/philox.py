"""Philox4x32-10 counter-based generator and the uniform/Gumbel maps of the
sampler's random protocol — oracle side (test infrastructure only).

Philox4x32-10 as defined in Salmon, Moraes, Dror and Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3" (SC'11): a 4-word counter and a 2-word key;
each of the 10 rounds multiplies counter words 0 and 2 by two fixed 32-bit
constants, forms the next counter from the high/low halves of the products
xor-ed with the other two words and the round key, and the key advances by two
Weyl constants between rounds.

Written with plain numpy uint64 arithmetic (a 32x32-bit product fits in 64
bits), vectorised over counters. Shares no code with the HIP implementation.
Pinned by: the Random123 known-answer vectors (tests/golden) and PyTorch's own
ATen Philox engine (tests/test_oracle_philox.py), plus a chi-square test of the
uniform map.
"""
import numpy as np

MULT_0 = np.uint64(0xD2511F53)
MULT_1 = np.uint64(0xCD9E8D57)
WEYL_0 = np.uint64(0x9E3779B9)
WEYL_1 = np.uint64(0xBB67AE85)
_LOW32 = np.uint64(0xFFFFFFFF)
_SHIFT32 = np.uint64(32)

# Counter word 3 of every draw says what the draw is for.
TAG_INIT = 0      # initial canvas token
TAG_BLOCK = 1     # block-level Gumbel noise of the sample
TAG_ELEM = 2      # element-level Gumbel noise inside the chosen block
TAG_RENOISE = 3   # uniform token at a non-accepted position
TAG_CANVAS = 4    # seed of a later canvas of a block-autoregressive stream


def _u32(x):
    return np.asarray(x, dtype=np.uint64) & _LOW32


def philox4x32_10(ctr0, ctr1, ctr2, ctr3, key0, key1):
    """Return the four 32-bit output words (as uint64 arrays) of Philox4x32-10
    for the given counter words and key words (broadcast together)."""
    c0, c1, c2, c3 = _u32(ctr0), _u32(ctr1), _u32(ctr2), _u32(ctr3)
    k0, k1 = _u32(key0), _u32(key1)
    c0, c1, c2, c3, k0, k1 = np.broadcast_arrays(c0, c1, c2, c3, k0, k1)
    for _ in range(10):
        prod0 = c0 * MULT_0
        prod1 = c2 * MULT_1
        hi0, lo0 = prod0 >> _SHIFT32, prod0 & _LOW32
        hi1, lo1 = prod1 >> _SHIFT32, prod1 & _LOW32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
        k0 = (k0 + WEYL_0) & _LOW32
        k1 = (k1 + WEYL_1) & _LOW32
    return c0, c1, c2, c3


def seed_key(seed):
    """Key words of a canvas seed (uint64): (low 32 bits, high 32 bits)."""
    s = int(seed) & 0xFFFFFFFFFFFFFFFF
    return s & 0xFFFFFFFF, s >> 32


def uniform_open01(word):
    """U = (2*(w >> 9) + 1) / 2^24: 23 random bits, strictly inside (0, 1),
    exactly representable in fp32 and fp64."""
    w = np.asarray(word, dtype=np.uint64)
    return ((w >> np.uint64(9)).astype(np.float64) * 2.0 + 1.0) * 2.0 ** -24


def gumbel(word):
    """Standard Gumbel variate -ln(-ln U) of a 32-bit word, in fp64."""
    return -np.log(-np.log(uniform_open01(word)))


def uniform_token(word, vocab):
    """floor(w * V / 2^32): a vocabulary id in [0, V) from a 32-bit word."""
    w = np.asarray(word, dtype=np.uint64)
    return ((w * np.uint64(vocab)) >> _SHIFT32).astype(np.int64)
