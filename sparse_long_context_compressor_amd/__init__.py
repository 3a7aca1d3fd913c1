"""MI355X-native compressed sparse attention layer (DeepSeek-V4 style).

The compute lives in a C-ABI shared library of hand-written HIP kernels for
gfx950 (``csrc/``, built to ``libslc.so``); ``slc`` is its thin Python binding
(argument marshalling only).  ``pools`` describes the paged pool layouts and
``inputs`` draws seeded synthetic workloads.
"""
__all__ = ["slc", "pools", "inputs"]
