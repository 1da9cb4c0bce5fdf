"""MI355X-native Multi-head Latent Attention over a paged latent cache.

The compute lives in ``libmla.so`` (hand-written HIP for gfx950, C ABI in
``include/mla.h``); :mod:`mla_latent_kv_22_amd.mla` is the thin ctypes
binding.  Importing this package loads nothing; the library is opened on the
first call.
"""
__all__ = ["inputs", "mla"]
