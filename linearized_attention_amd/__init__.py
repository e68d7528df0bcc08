"""Lizard attention for AMD MI355X (gfx950).

The compute path is the C-ABI library ``liblizard_attn.so`` (hand-written HIP
kernels, declared in ``include/lizard_attn.h``).  ``api`` is a thin ctypes
binding that marshals torch tensors into it; nothing here computes attention
on the CPU.  ``synthetic`` draws the seeded inputs used by tests and the
benchmark.
"""
__all__ = ["api", "synthetic"]
