"""libfairy for AMD MI355X: the multiplication-free 2-bit complex linear layer.

The compute path lives in the HIP shared library ``libfairy.so`` (C ABI,
declared in include/fairy.h).  ``bit_complex_weight_amd.fairy`` is a thin
ctypes binding with the same entry-point names; it does argument marshalling
only and raises if the library is missing -- there is no CPU fallback.
"""
__all__ = ["fairy", "synth"]
