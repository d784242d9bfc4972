"""Plain fp64 CPU implementation of one step and of the whole denoising loop of
the canvas sampler — the oracle (test infrastructure only).

Rules, as the pages state them:
  "DiffusionGemma Lab" (shadowgraph.io), §2 "The generation algorithm, as
  written in the code":
    item 1  the canvas starts as uniform random vocabulary tokens, not [MASK];
    item 2  sort positions by entropy ascending, commit the largest prefix with
            cumsum(H) - max(H) <= 0.1 (always at least one position);
    item 3  stop when the argmax canvas is unchanged from the previous step
            and the mean entropy is below 0.005;
    item 4  temperature goes linearly from 0.8 to 0.4 across steps;
    item 5  (garbled on the page) read as: a run returns its argmax canvas,
            and a committed position takes that step's multinomial draw.
  "DiffusionGemma: Parallel Denoising From an Autoregressive Checkpoint"
  (boxwrench.dev), "Finding", Algorithm 1: multinomial (uniform-noise)
  diffusion; the non-accepted remainder is renoised uniformly; the budget is
  N = 48 steps.

Where the pages are silent the readings are: entropy of the tempered softmax
in nats; argmax of the raw logits, lowest id on ties; sort ties broken by
position; acceptance is per step (nothing is frozen across steps); renoise
draws uniformly over all of [0, V); the stop needs a previous step; the
temperature schedule clamps after its last step. The multinomial sample is
drawn with a fixed two-level Gumbel-max protocol (below) so that a second
implementation can reproduce it bit for bit.

Everything is numpy float64 on the exact input values (bf16 and fp32 widen to
fp64 exactly). Shares no code with the HIP implementation.
"""
import numpy as np

from .philox import (TAG_BLOCK, TAG_ELEM, TAG_INIT, TAG_RENOISE, gumbel,
                     philox4x32_10, seed_key, uniform_token)

# Vocabulary geometry of the sampling protocol: a stripe is 512 consecutive
# ids cut into 64 slots of 8; a chunk is 8 consecutive stripes; a block is one
# slot taken across the 8 stripes of a chunk (up to 64 ids). Any partition of
# the ids into blocks gives an exact sample; this one is the protocol.
SLOT_IDS = 8
SLOTS = 64
STRIPE_IDS = SLOT_IDS * SLOTS        # 512
CHUNK_STRIPES = 8
CHUNK_IDS = STRIPE_IDS * CHUNK_STRIPES   # 4096


# ----------------------------------------------------------------------------
# Schedule — "DiffusionGemma Lab" §2 item 4; boxwrench.dev Algorithm 1,
# temperature annealing (linear 0.8 -> 0.4 across the denoising steps).
# ----------------------------------------------------------------------------
def temperature(step, t_start=0.8, t_end=0.4, n_sched=48):
    """T at `step`: linear from t_start (step 0) to t_end (step n_sched-1),
    held at t_end afterwards; evaluated in double, rounded once to fp32."""
    t0 = float(np.float32(t_start))
    t1 = float(np.float32(t_end))
    if n_sched == 1:
        return np.float32(t0)
    frac = min(step, n_sched - 1) / (n_sched - 1)
    return np.float32(t0 + (t1 - t0) * frac)


# ----------------------------------------------------------------------------
# Per-position statistics — "DiffusionGemma Lab" §2 items 2, 4, 5.
# ----------------------------------------------------------------------------
def entropy(z, temp):
    """Entropy in nats of softmax(z / T) for each row of z ([rows, V]):
    H = -sum_{p > 0} p ln p, clamped to +0."""
    x = np.asarray(z, dtype=np.float64) / np.float64(temp)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    p = e / np.sum(e, axis=-1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        terms = np.where(p > 0, -p * np.log(np.where(p > 0, p, 1.0)), 0.0)
    h = np.sum(terms, axis=-1)
    return np.where(h > 0, h, 0.0)


def argmax_raw(z):
    """Lowest vocabulary id attaining the maximum raw logit, per row."""
    return np.argmax(np.asarray(z), axis=-1).astype(np.int64)


def block_index(v):
    """Block of vocabulary id v: 64 * chunk + slot."""
    v = np.asarray(v, dtype=np.int64)
    return SLOTS * (v // CHUNK_IDS) + (v // SLOT_IDS) % SLOTS


def block_members(j, vocab):
    """Vocabulary ids of block j in increasing order (ids >= V dropped)."""
    chunk, slot = divmod(int(j), SLOTS)
    stripe = np.arange(CHUNK_STRIPES, dtype=np.int64)[:, None]
    elem = np.arange(SLOT_IDS, dtype=np.int64)[None, :]
    v = (chunk * CHUNK_IDS + stripe * STRIPE_IDS + slot * SLOT_IDS + elem).ravel()
    return v[v < vocab]


def block_word(j, pos, step, k0, k1):
    """Random word of block j's Gumbel: one Philox call serves the four blocks
    that differ only in bits 9-10 of j (chunks 8 apart), block j taking word
    (j >> 9) & 3 of the call with counter c0 = j with those bits cleared."""
    j = np.asarray(j, dtype=np.int64)
    words = philox4x32_10(j & ~0x600, pos, step, TAG_BLOCK, k0, k1)
    return np.choose((j >> 9) & 3, words)


def block_logsumexp(x):
    """Log-sum-exp of x (fp64, [rows, V], already divided by T) over every
    block; result [rows, n_blocks] indexed by block number (empty -> -inf)."""
    rows, vocab = x.shape
    n_chunk = -(-vocab // CHUNK_IDS)
    pad = np.full((rows, n_chunk * CHUNK_IDS), -np.inf)
    pad[:, :vocab] = x
    # axes: row, chunk, stripe within chunk, slot, id within slot
    xb = pad.reshape(rows, n_chunk, CHUNK_STRIPES, SLOTS, SLOT_IDS)
    m = np.max(xb, axis=(2, 4))                       # [rows, n_chunk, slot]
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    s = np.sum(np.exp(xb - m_safe[:, :, None, :, None]), axis=(2, 4))
    with np.errstate(divide="ignore"):
        lse = np.where(finite, m_safe + np.log(s), -np.inf)
    return lse.reshape(rows, n_chunk * SLOTS)


def sample_two_level_detail(z, temp, seed, positions, step):
    """Multinomial sample of softmax(z/T) per row by the two-level Gumbel-max
    protocol: block j* = argmax_j (LSE_j + G_j), then the id inside j* with the
    largest z_v/T + G_v. Ties go to the lowest block, then the lowest id. Exact
    in distribution by the Gumbel-max property applied twice.

    z: [rows, V]; positions: [rows] canvas positions (counter word 1).
    Returns (samples, block_best, block_gap, elem_best, elem_gap): the winning
    scores of both levels and their margins over the runner-up (inf when there
    is none), used to recognise near-ties between implementations."""
    x = np.asarray(z, dtype=np.float64) / np.float64(temp)
    rows, vocab = x.shape
    k0, k1 = seed_key(seed)
    lse = block_logsumexp(x)
    n_blocks = lse.shape[1]
    j = np.arange(n_blocks, dtype=np.int64)[None, :]
    pos = np.asarray(positions, dtype=np.int64)[:, None]
    block_score = lse + gumbel(block_word(j, pos, step, k0, k1))
    j_star = np.argmax(block_score, axis=1)
    out = np.empty(rows, dtype=np.int64)
    detail = np.full((4, rows), np.inf)
    for r in range(rows):
        v = block_members(j_star[r], vocab)
        words = philox4x32_10(v >> 2, positions[r], step, TAG_ELEM, k0, k1)
        w = np.choose(v & 3, words)
        score = x[r, v] + gumbel(w)
        out[r] = v[np.argmax(score)]
        top_b = np.sort(block_score[r])[::-1]
        top_e = np.sort(score)[::-1]
        detail[0, r] = top_b[0]
        detail[2, r] = top_e[0]
        if len(top_b) > 1:
            detail[1, r] = top_b[0] - top_b[1]
        if len(top_e) > 1:
            detail[3, r] = top_e[0] - top_e[1]
    return (out,) + tuple(detail)


def sample_two_level(z, temp, seed, positions, step):
    """Multinomial sample per row by the two-level Gumbel-max protocol (see
    sample_two_level_detail)."""
    return sample_two_level_detail(z, temp, seed, positions, step)[0]


def sample_per_element(z, temp, seed, positions, step):
    """Reference variant for distribution tests only: plain Gumbel-max over
    every id with the element-level noise, argmax_v (z_v/T + G_v)."""
    x = np.asarray(z, dtype=np.float64) / np.float64(temp)
    rows, vocab = x.shape
    k0, k1 = seed_key(seed)
    v = np.arange(vocab, dtype=np.int64)
    out = np.empty(rows, dtype=np.int64)
    for r in range(rows):
        words = philox4x32_10(v >> 2, positions[r], step, TAG_ELEM, k0, k1)
        out[r] = np.argmax(x[r] + gumbel(np.choose(v & 3, words)))
    return out


# ----------------------------------------------------------------------------
# Per-canvas decisions — "DiffusionGemma Lab" §2 items 1-3;
# boxwrench.dev Algorithm 1 (entropy-bounded acceptance, adaptive stopping).
# ----------------------------------------------------------------------------
def accept(h, bound):
    """Sort positions by (entropy, position) ascending and accept the longest
    prefix whose cumulative entropy minus its largest entropy is <= bound.
    Returns (accepted mask [L] bool, number accepted)."""
    h = np.asarray(h, dtype=np.float64)
    L = h.shape[0]
    order = np.lexsort((np.arange(L), h))
    hs = h[order]
    ok = (np.cumsum(hs) - np.maximum.accumulate(hs)) <= np.float64(bound)
    k = L if ok.all() else int(np.argmin(ok))
    mask = np.zeros(L, dtype=bool)
    mask[order[:k]] = True
    return mask, k


def uniform_tokens(seed, canvas_len, step, vocab, tag):
    """One uniform vocabulary id per position from word 0 of (0, l, step, tag)."""
    k0, k1 = seed_key(seed)
    w0 = philox4x32_10(0, np.arange(canvas_len), step, tag, k0, k1)[0]
    return uniform_token(w0, vocab)


def init_canvas(seed, canvas_len, vocab):
    """Initial canvas: uniform random tokens ("DiffusionGemma Lab" §2 item 1)."""
    return uniform_tokens(seed, canvas_len, 0, vocab, TAG_INIT)


def stop_test(argmax, prev_argmax, mean_h, threshold):
    """Adaptive stop: a previous argmax canvas exists, it equals this step's at
    every position, and the mean entropy is strictly below the threshold."""
    stable = prev_argmax is not None and bool(np.array_equal(argmax, prev_argmax))
    return stable and bool(mean_h < np.float64(threshold))


def row_statistics(z, temp, seed, positions, step_index):
    """Per-row statistics of one step for rows z ([rows, V], any float dtype,
    widened exactly to fp64) at canvas positions `positions`: entropy, raw
    argmax and the two-level sample, with the sample's winning scores and
    margins at both levels (see sample_two_level_detail)."""
    z = np.asarray(z, dtype=np.float64)
    smp, bbest, bgap, ebest, egap = sample_two_level_detail(z, temp, seed, positions, step_index)
    return dict(entropy=entropy(z, temp), argmax=argmax_raw(z), sample=smp,
                block_best=bbest, block_gap=bgap, elem_best=ebest, elem_gap=egap)


def decide(h, am, smp, seed, step_index, vocab, prev_argmax=None, bound=np.float32(0.1),
           stop_threshold=np.float32(0.005)):
    """The per-canvas decisions of one step from its rows' entropies h,
    argmaxes am and samples smp ([L] each): acceptance, the new canvas
    (accepted positions take the sample, the rest a fresh uniform token), the
    mean entropy and the stop."""
    h = np.asarray(h, dtype=np.float64)
    mask, k = accept(h, bound)
    renoise = uniform_tokens(seed, h.shape[0], step_index, vocab, TAG_RENOISE)
    canvas = np.where(mask, smp, renoise)
    mean_h = float(np.mean(h))
    stop = stop_test(am, prev_argmax, mean_h, stop_threshold)
    return dict(accept=mask, n_accept=k, canvas=canvas, renoise=renoise, mean_entropy=mean_h,
                stop=stop)


def step(z, temp, seed, step_index, prev_argmax=None, bound=np.float32(0.1),
         stop_threshold=np.float32(0.005), rows_per_chunk=16):
    """One sampler step over one canvas. z: [L, V] logits (any float dtype,
    widened exactly to fp64). Returns a dict of every step output."""
    z = np.asarray(z)
    L, vocab = z.shape
    parts = [row_statistics(z[r0:r0 + rows_per_chunk], temp, seed,
                            np.arange(r0, min(r0 + rows_per_chunk, L)), step_index)
             for r0 in range(0, L, rows_per_chunk)]
    out = {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}
    out.update(decide(out["entropy"], out["argmax"], out["sample"], seed, step_index, vocab,
                      prev_argmax, bound, stop_threshold))
    return out


def run(denoise, seed, canvas_len, vocab, t_start=0.8, t_end=0.4, n_sched=48,
        max_steps=48, bound=np.float32(0.1), stop_threshold=np.float32(0.005),
        record=False):
    """Whole denoising of one canvas: init, then up to max_steps steps; the
    output is the argmax canvas of the step where the stop fires, else of the
    last step. denoise(step, canvas) -> logits [L, V].
    Returns (final argmax, steps used, stopped, per-step records or None)."""
    canvas = init_canvas(seed, canvas_len, vocab)
    prev = None
    records = [] if record else None
    for s in range(max_steps):
        z = denoise(s, canvas)
        out = step(z, temperature(s, t_start, t_end, n_sched), seed, s, prev,
                   bound, stop_threshold)
        if record:
            records.append(dict(out, canvas_in=canvas))
        if out["stop"]:
            return out["argmax"], s + 1, True, records
        prev = out["argmax"]
        canvas = out["canvas"]
    return prev, max_steps, False, records
