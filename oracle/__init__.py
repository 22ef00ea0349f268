"""CPU oracle for quantized-KV attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import this package.  The product
library (``quantized_kv_cache_amd``) never imports it and has no CPU fallback.

The arithmetic lives in ``qkv_oracle.c`` (plain C, fp64 attention), loaded
through ctypes by :mod:`oracle.oracle`.  Nothing here is shared with the GPU
path.
"""
from .oracle import *  # noqa: F401,F403
