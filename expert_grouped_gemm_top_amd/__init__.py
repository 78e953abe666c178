"""MI355X-native MoE expert hot path: top-k routing, counting-sort dispatch,
SwiGLU experts as variable-size grouped GEMMs, router-weighted combine, and the
backward (dx, dW) over an optionally compacted set of retained pairs.

The compute lives in ``libmoe.so`` (hand-written HIP for gfx950 behind a C ABI,
declared in ``include/moe.h``); ``expert_grouped_gemm_top_amd.moe`` is the thin
ctypes binding.  Importing this package does not load the library; the first
call does, and fails loudly if it has not been built.
"""
