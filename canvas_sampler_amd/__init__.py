"""MI355X (gfx950) canvas sampler for block-diffusion decoding.

The compute path is the HIP library libdgcanvas.so (C ABI in include/dg_canvas.h);
`canvas_sampler_amd.binding` marshals arguments to it and nothing else.
`canvas_sampler_amd.synth` generates seeded synthetic inputs.
"""
__all__ = ["binding", "synth"]
