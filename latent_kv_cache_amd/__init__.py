"""MI355X-native GQLA decode attention.

The compute path is the C-ABI library ``libgqla.so`` (hand-written HIP for
gfx950) declared in ``include/gqla.h``; ``latent_kv_cache_amd.gqla`` is its
thin ctypes binding.  ``roofline`` is host-side bookkeeping for measurement.
"""
