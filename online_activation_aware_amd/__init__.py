"""libttq: activation-aware test-time quantization (TTQ) on MI355X (gfx950).

The per-prompt hot path of one linear layer — activation statistics, shrunk
AWQ scales, group-wise RTN of the scaled weight, and the quantized projection
(plus an optional low-rank term) — runs as hand-written HIP kernels behind a
C ABI (``include/ttq.h``).  ``online_activation_aware_amd.ttq`` is the thin
Python binding; importing this package does not load the library.
"""
__all__ = ["ttq", "synth"]
