"""fp64 CPU oracle for the KDA chunked forward -- test infrastructure only.

Only the test suite, the smoke check and the CPU-baseline leg of the benchmark may import
this package.  The GPU library and its Python binding never import it.

The arithmetic lives in ``kda_oracle.c`` (plain C, fp64, OpenMP over independent state-row
chains).  This module only builds that file with gcc and marshals arrays through ctypes.
"""
from .oracle import (  # noqa: F401
    LAYOUTS,
    QK_L2NORM,
    BETA_SIGMOID,
    SCALAR_GATE,
    build_oracle,
    load_oracle,
    kda_oracle,
    oracle_threads,
)
