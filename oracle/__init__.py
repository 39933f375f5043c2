"""fp64 CPU oracle for exact attention.

TEST INFRASTRUCTURE ONLY: the checker the GPU path is compared against.  Only
tests/, the smoke check in __graft_entry__ and the CPU-baseline leg of bench.py
may import it.  It shares no code with the HIP library and the library never
calls it.
"""
from .oracle import (Oracle, attention, attention_bwd, attention_bwd_rows, attention_online,  # noqa: F401
                     attention_rows, build, compile_source, library_path, num_threads, source_text)
from . import attn_matmul  # noqa: F401  (whole-matrix fp64 oracle for full-size checks)
