"""MI355X-native InfLLM context-memory attention step.

The work is done by ``libinfllm.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/infllm.h``); ``block_level_kv_amd.infllm`` is the thin
ctypes binding with the same call names.  Importing the package loads
nothing; the binding loads the library on first use and raises if it is
missing.
"""
__all__ = ["synth", "infllm"]
