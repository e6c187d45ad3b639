"""MI355X-native quantized KV cache and decode attention (libkvq).

The compute path is the HIP library ``libkvq.so`` (C ABI in include/kvq.h);
``kvq`` is its ctypes binding.
"""
from . import kvq  # noqa: F401
