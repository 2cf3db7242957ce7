"""fp64 CPU attention oracle -- test infrastructure only.

Imported only by ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py``.  It shares no code with the GPU library.
"""
from .oracle import (Oracle, attention, attention_bwd, attention_decode,  # noqa: F401
                     attention_decode_paged, attention_fp8, attention_mod, attention_rows, attention_varlen, build,
                     decode_e4m3, default, load)
