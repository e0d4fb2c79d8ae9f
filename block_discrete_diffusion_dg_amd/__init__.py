"""One block-diffusion denoising step on MI355X (gfx950), behind a C ABI.

The compute path lives in ``libdg.so`` (hand-written HIP kernels, see
``csrc/``); ``binding`` marshals torch tensors into its C entry points and
``engine`` strings the calls into a block loop. Importing this package loads
nothing native: the library is opened on first use and a missing library is an
error, never a fallback.
"""
__all__ = ["synth"]
