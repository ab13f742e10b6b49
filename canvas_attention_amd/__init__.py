"""MI355X (gfx950) canvas denoising attention.

The GPU path lives in libdg.so (HIP kernels behind the C ABI of include/dg.h);
``canvas_attention_amd.dg`` is its Python binding and ``canvas_attention_amd.synth``
draws the seeded synthetic inputs.  Build with ``python -m canvas_attention_amd.build``.
"""
__all__ = ["dg", "synth", "build"]
