"""MI355X-native (gfx950) forward pass of a sparse Mixture-of-Experts layer.

The computation lives in the HIP library ``libmoe.so`` (C ABI, declared in
``include/moe.h``); ``sparse_mixture_experts_level_amd.ops`` is its thin
Python binding.  Importing this package loads nothing; the library is loaded,
and must be present, on the first call into the binding.
"""
__all__ = ["ops", "workloads"]
