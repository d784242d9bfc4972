"""dg_sampler_step_noalloc (the step for callers that cannot allocate) against
dg_sampler_step through the C ABI: every output equal bit for bit, on two
calls in a row of which the second is smaller (the static scratch keeps the
first call's contents), including a batch small enough to split each row over
several workgroups; sizes beyond the static scratch are rejected before
anything is written."""
import numpy as np
import pytest
import torch

from canvas_sampler_amd import binding as B
from canvas_sampler_amd import synth

from gpu_util import gpu, require_gpu, seeds_tensor

pytestmark = gpu


def _bufs(n, Bn):
    return dict(canvas_out=torch.full((n,), -3, dtype=torch.int32, device="cuda"),
                argmax_out=torch.full((n,), -3, dtype=torch.int32, device="cuda"),
                sample_out=torch.full((n,), -3, dtype=torch.int32, device="cuda"),
                accept_out=torch.full((n,), 9, dtype=torch.uint8, device="cuda"),
                entropy_out=torch.full((n,), -3.0, device="cuda"),
                n_accept_out=torch.full((Bn,), -3, dtype=torch.int32, device="cuda"),
                mean_entropy_out=torch.full((Bn,), -3.0, device="cuda"),
                stop_out=torch.full((Bn,), 9, dtype=torch.uint8, device="cuda"))


def _case(L, V, Bn, dtype, gen, step):
    z = torch.cat([synth.sharpening_logits(gen + c, step, L, V, m0_max=6.0, dtype=dtype, device="cuda")
                   for c in range(Bn)])
    params = B.params_default(canvas_len=L, vocab=V, temp_steps=16)
    temps = torch.tensor([B.dg_temperature(params, step + c) for c in range(Bn)], device="cuda")
    seeds = seeds_tensor([gen * 7 + c for c in range(Bn)])
    prev = torch.randint(0, V, (Bn * L,), dtype=torch.int32, device="cuda")
    return params, z, temps, seeds, prev


def test_noalloc_step_equals_sampler_step_on_two_calls():
    require_gpu()
    # first a large call (3 canvases x 256 rows, ragged V, one workgroup per
    # row), then a smaller one (one canvas of 40 rows: each row split over
    # two workgroups, so the static partials and the merge kernel are used),
    # then the large one again
    cases = [(256, 70001 + 7, 3, torch.bfloat16, 11, 4), (40, 4096 * 96, 1, torch.float32, 23, 2),
             (256, 70001 + 7, 3, torch.bfloat16, 11, 4)]
    for L, V, Bn, dtype, gen, step in cases:
        V = V - V % 8
        params, z, temps, seeds, prev = _case(L, V, Bn, dtype, gen, step)
        want = _bufs(Bn * L, Bn)
        ctx = B.Context(params, max_batch=Bn)
        ctx.dg_sampler_step(z, temps, step, seeds, ctx.step_out(**want), prev_argmax=prev)
        got = _bufs(Bn * L, Bn)
        B.sampler_step_noalloc(params, z, temps, step, seeds, B.Context.step_out(**got), prev_argmax=prev)
        # and with the statistics left in the static scratch
        lean = _bufs(Bn * L, Bn)
        B.sampler_step_noalloc(params, z, temps, step, seeds,
                               B.Context.step_out(canvas_out=lean["canvas_out"], n_accept_out=lean["n_accept_out"],
                                                  stop_out=lean["stop_out"]), prev_argmax=prev)
        torch.cuda.synchronize()
        for k in want:
            assert torch.equal(want[k], got[k]), f"L={L} V={V} B={Bn}: {k} differs"
        for k in ("canvas_out", "n_accept_out", "stop_out"):
            assert torch.equal(want[k], lean[k]), f"L={L} V={V} B={Bn}: {k} differs (statistics in scratch)"
        assert int(want["n_accept_out"].min()) >= 1
        ctx.close()
        print(f"L={L} V={V} B={Bn} {dtype}: equal; commits {want['n_accept_out'].tolist()}")


def test_noalloc_rejects_batches_beyond_the_static_scratch():
    require_gpu()
    L, V = 256, 4096
    params = B.params_default(canvas_len=L, vocab=V)
    Bn = 16384 // L + 1
    z = torch.zeros(Bn * L, V, device="cuda")
    temps = torch.full((Bn,), 0.8, device="cuda")
    seeds = seeds_tensor(list(range(Bn)))
    out = _bufs(Bn * L, Bn)
    with pytest.raises(B.DgError) as e:
        B.sampler_step_noalloc(params, z, temps, 0, seeds, B.Context.step_out(**out))
    assert e.value.status == B.DG_ERR_INVALID_ARG and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.all(out["canvas_out"] == -3) and torch.all(out["stop_out"] == 9)
    # the largest batch it takes still runs
    Bn -= 1
    out = _bufs(Bn * L, Bn)
    B.sampler_step_noalloc(params, z[:Bn * L], temps[:Bn], 0, seeds[:Bn], B.Context.step_out(**out))
    torch.cuda.synchronize()
    # constant logits: every entropy is ln V and exactly one position commits
    assert torch.all(out["n_accept_out"] == 1)
    assert np.allclose(out["entropy_out"].cpu().numpy(), np.log(V), atol=1e-4)
