"""fp64 CPU oracle for sliding-window attention with sinks.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``.  The product package never
imports it, and it imports nothing from the product package.
"""
from .oracle import (  # noqa: F401
    RollingCacheSim,
    attend_set,
    backward,
    build,
    chunked_rows,
    decode_row,
    key_set,
    library_path,
    prefill_rows,
    rope,
    threads,
)
