"""CPU oracle for the 2-bit mixed-precision KV cache (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package; the product library never does.  Its only parity pins are the tests
under ``tests/`` that check it against what the pages and the mathematics fix.
"""
from .oracle import (BF16, D, F16, GK, GV, P, R, OracleCache, OracleLib, lib,  # noqa: F401
                     planted)
