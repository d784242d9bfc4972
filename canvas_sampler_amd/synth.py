"""Seeded synthetic inputs for the canvas sampler: stand-ins for a denoiser's
logits and for LM-head operands, shaped like the pages' workload (canvases of
256 positions, a 262,144-token vocabulary, 12-48 steps).

This module only generates numbers; it holds none of the sampler's arithmetic.
Tests feed the very same tensor bits to the HIP library and to the oracle, so
the generator's own accuracy does not matter. Values come from torch's seeded
generators on the requested device (CPU and GPU streams differ; that is fine
because both sides always consume one tensor).

Workloads:
  margin_logits       one step: iid N(0,1) plus a margin m ~ U[0, m_max] at a
                      uniformly drawn target id per position.
  sharpening_logits   a denoiser whose confidence grows: fixed target id and
                      base margin m0 ~ U[0, m0_max] per position; at step s the
                      logits are fresh iid N(0,1) plus m0 + growth * s at the
                      target ("DiffusionGemma Lab", EXP B: synthetic logits
                      whose confidence ramps over steps, per-position
                      difficulty).
  chained_targets,    block-autoregressive stand-in: canvas k of a stream has
  chained_logits      per-position targets that continue the previous finished
                      canvas (target_l = (prev_{(l+1) mod L} + shift_k) mod V,
                      shift_k drawn per canvas; canvas 0 draws them uniformly)
                      and sharpens on them like sharpening_logits ("DiffusionGemma
                      Lab", Figure 1: finished canvases chain block-autoregressively).
  iid_normal_logits   untrained-model stand-in: iid N(0, variance), fresh each
                      step, no margin ("DiffusionGemma Lab", EXP A).
  lmhead_operands     hidden states N(0,1) and weights N(0, 1/K) in bf16, so
                      that logits = hidden @ weight are about unit scale.
  selfcond_embedding  fp32 [V, d] ~ N(0,1): synthetic parameters of the
                      self-conditioning matmul (7.86 M at V = 262144, d = 30).
"""
import torch

_MIX = 0x9E3779B97F4A7C15
_MASK63 = (1 << 63) - 1


def _gen(device, *parts):
    """torch.Generator on `device` seeded from a tuple of integers."""
    h = 0x243F6A8885A308D3
    for p in parts:
        h = ((h ^ (int(p) & 0xFFFFFFFFFFFFFFFF)) * _MIX + 0x632BE59BD9B4E019) & 0xFFFFFFFFFFFFFFFF
        h ^= h >> 29
    g = torch.Generator(device=device)
    g.manual_seed(h & _MASK63)
    return g


def _targets_and_margins(gen_seed, canvas_len, vocab, m_max, device):
    g = _gen(device, gen_seed, 0xA11CE)
    target = torch.randint(0, vocab, (canvas_len,), generator=g, device=device)
    margin = torch.rand(canvas_len, generator=g, device=device, dtype=torch.float32) * m_max
    return target, margin


def _finish(z, target, add, dtype, out):
    rows = torch.arange(z.shape[0], device=z.device)
    z[rows, target] += add
    if out is None:
        return z.to(dtype)
    out.copy_(z)  # rounds to out.dtype (round-to-nearest-even for bf16)
    return out


def margin_logits(gen_seed, canvas_len, vocab, m_max=12.0, dtype=torch.float32,
                  device="cpu", out=None):
    """Single-step logits: N(0,1) plus m ~ U[0, m_max] at a target id."""
    target, margin = _targets_and_margins(gen_seed, canvas_len, vocab, m_max, device)
    g = _gen(device, gen_seed, 0xB0B)
    z = torch.randn(canvas_len, vocab, generator=g, device=device, dtype=torch.float32)
    return _finish(z, target, margin, dtype, out)


def sharpening_logits(gen_seed, step, canvas_len, vocab, m0_max=6.0, growth=1.5,
                      dtype=torch.bfloat16, device="cpu", out=None):
    """Step `step` of the sharpening denoiser: N(0,1) + (m0 + growth*step) at
    the per-position target; targets and m0 are fixed for a gen_seed."""
    target, m0 = _targets_and_margins(gen_seed, canvas_len, vocab, m0_max, device)
    g = _gen(device, gen_seed, 0x5EED, step)
    z = torch.randn(canvas_len, vocab, generator=g, device=device, dtype=torch.float32)
    return _finish(z, target, m0 + growth * step, dtype, out)


def chained_targets(gen_seed, canvas_index, prev_canvas, canvas_len, vocab, m0_max=6.0,
                    device="cpu"):
    """(target ids [L] int64, base margins m0 [L]) of canvas `canvas_index` of
    the block-autoregressive stand-in; prev_canvas: the previous finished
    canvas (tensor [L] on `device`), None for canvas 0."""
    g = _gen(device, gen_seed, 0xC4A1, canvas_index)
    m0 = torch.rand(canvas_len, generator=g, device=device, dtype=torch.float32) * m0_max
    if prev_canvas is None:
        target = torch.randint(0, vocab, (canvas_len,), generator=g, device=device)
    else:
        shift = torch.randint(1, vocab, (1,), generator=g, device=device)
        target = (torch.roll(prev_canvas.to(device=device, dtype=torch.int64), -1) + shift) % vocab
    return target, m0


def chained_logits(gen_seed, canvas_index, step, target, m0, vocab, growth=1.5,
                   dtype=torch.bfloat16, device="cpu", out=None):
    """Step `step` of canvas `canvas_index`: fresh N(0,1) plus m0 + growth*step
    at the targets from chained_targets."""
    g = _gen(device, gen_seed, 0xC4A2, canvas_index, step)
    z = torch.randn(target.shape[0], vocab, generator=g, device=device, dtype=torch.float32)
    return _finish(z, target, m0 + growth * step, dtype, out)


def iid_normal_logits(gen_seed, step, canvas_len, vocab, variance=0.05,
                      dtype=torch.float32, device="cpu", out=None):
    """Step `step` of the untrained-model stand-in: iid N(0, variance)."""
    g = _gen(device, gen_seed, 0x1DD, step)
    z = torch.randn(canvas_len, vocab, generator=g, device=device, dtype=torch.float32)
    z *= variance ** 0.5
    if out is None:
        return z.to(dtype)
    out.copy_(z)
    return out


def lmhead_operands(gen_seed, rows, k, vocab, device="cpu"):
    """hidden bf16 [rows, k] ~ N(0,1); weight bf16 [k, vocab] ~ N(0, 1/k)."""
    g = _gen(device, gen_seed, 0x4EAD)
    hidden = torch.randn(rows, k, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)
    weight = torch.empty(k, vocab, device=device, dtype=torch.bfloat16)
    chunk = max(1, (1 << 26) // vocab)
    for k0 in range(0, k, chunk):
        part = torch.randn(min(chunk, k - k0), vocab, generator=g, device=device,
                           dtype=torch.float32)
        weight[k0:k0 + part.shape[0]] = (part * (1.0 / k) ** 0.5).to(torch.bfloat16)
    return hidden, weight


def selfcond_embedding(gen_seed, vocab, d=30, device="cpu"):
    """fp32 [vocab, d] ~ N(0, 1)."""
    g = _gen(device, gen_seed, 0x5C0D)
    return torch.randn(vocab, d, generator=g, device=device, dtype=torch.float32)
