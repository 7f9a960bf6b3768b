"""CPU oracle for one DSA layer (fp64, NumPy) -- TEST INFRASTRUCTURE.

Only tests, the smoke check and the CPU-baseline leg of the benchmark may
import anything under this directory.  The product path (the HIP library and
its Python binding) never does, and this package imports nothing from it.

Parity status of each function is listed with its pins in tests/test_oracle.py
(the front-end quantisers of quant.py: tests/test_oracle_quant.py; the sharded
top-k merge of merge.py: tests/test_oracle_merge.py):
every function here is pinned by closed forms, invariants, library routines or
brute force on tiny inputs; the absolute values on random inputs are fixed only
through those pins (the pages print no worked DSA example).
"""
from . import codecs, dsa, merge, msa, quant  # noqa: F401
