"""SRFT-rotated low-bit KV-cache quantization and fused decode attention for MI355X (gfx950).

The compute path is the C-ABI library ``libkvq.so`` (hand-written HIP kernels); this package
only holds its Python binding (``kv_cache_quantization_srft_amd.kvq``) and seeded synthetic
inputs (``kv_cache_quantization_srft_amd.synth``).  Importing the package does not load the
library; the first call into ``kvq`` does, and fails loudly if it has not been built.
"""
__all__ = ["kvq", "synth"]
