"""MI355X-native rotated INT2 KV-cache quantization and decode attention.

The hot path lives in libkvq.so (hand-written HIP kernels for gfx950, C ABI in
include/kvq.h); ``decode_attention_int2_amd.kvq`` is its ctypes binding.  The
library is loaded on first use and there is no CPU fallback.
"""
from . import kvq  # noqa: F401

__all__ = ["kvq"]
