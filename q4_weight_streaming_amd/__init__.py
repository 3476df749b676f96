"""q4_weight_streaming_amd -- Q4_0-weight x Q8_0-activation weight-streaming GEMV for MI355X.

The compute runs in the HIP library ``libq4stream.so`` (gfx950); the Python
layer only marshals arguments through its C ABI (``include/q4s.h``).  The
library is loaded on first use, and every entry point raises if it is missing.
"""
__all__ = ["synth"]
