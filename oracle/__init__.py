"""TEST INFRASTRUCTURE ONLY: the fp64 CPU oracle of the KDA forward prefill.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package; the library path must never route through it. It shares no code
with the GPU library. Parity status of each function is listed in
reference.py's docstrings; every function here is pinned by tests in
tests/test_oracle_pins.py (none is "parity unpinned").
"""
from .reference import (recurrent, recurrent_c, dense, chunked, chunk_k1, chunk_k2,
                        segment_summary, build_c, c_max_threads, to_f64)

__all__ = ["recurrent", "recurrent_c", "dense", "chunked", "chunk_k1", "chunk_k2",
           "segment_summary", "build_c", "c_max_threads", "to_f64"]
