"""MI355X-native canvas denoising step (DiffusionGemma-style) over a C-ABI HIP library.

The compute lives in libdgstep.so (hand-written HIP for gfx950, built by
build.py); `binding` marshals arguments to it.  `synth` draws seeded inputs.
"""
__all__ = ["binding", "synth", "build"]
