"""MI355X (gfx950) sparse Mixture-of-Experts layer forward.

The compute path is the HIP library ``libmoe.so`` (C ABI declared in include/moe.h),
loaded by :mod:`sparse_mixture_experts_27_amd.binding`.  Importing this package does
not load the library; :func:`binding.lib` does, and raises if it is missing.
"""
__all__ = ["binding", "configs", "synth"]
