"""BeaconKV eviction step on MI355X (gfx950): HIP kernels behind a C ABI.

``reasoning_model_kv_amd.bkv`` is the ctypes binding of ``libbkv.so``
(see include/bkv.h); ``reasoning_model_kv_amd.build`` compiles it.
"""
