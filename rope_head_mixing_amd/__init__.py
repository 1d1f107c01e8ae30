"""MI355X-native fused inverse-RoPE + VHA postmix (forward, input grad, weight grad).

The compute path is hand-written HIP for gfx950 in ``csrc/`` behind a C-ABI
shared library (``libpostmix.so``, declared in ``include/postmix.h``).
``rope_head_mixing_amd.postmix`` is the thin ctypes binding with the same
entry-point names; it raises if the library is not built — there is no CPU
fallback.  ``rope_head_mixing_amd.synthetic`` holds the seeded input
generators.  Submodules are imported on demand so that importing the
generators never loads the GPU library.
"""

__all__ = ["postmix", "synthetic", "build"]
