"""KVarN hot path for MI355X (gfx950): HIP kernels behind a C ABI.

The native library ``libkvarn.so`` is loaded on first use by
:mod:`kv_cache_quantization_seal_amd.kvarn`; importing this package alone (for
example to use the synthetic workload generators) does not touch the GPU.
"""
__all__ = ["synth", "kvarn"]
