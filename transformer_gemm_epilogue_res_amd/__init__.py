"""MI355X (gfx950) fused GEMM -> residual -> RMSNorm -> GEMM chain, forward and backward.

The compute lives in libcoda.so (hand-written HIP, C ABI in include/coda.h);
this package is its thin binding plus the seeded synthetic-input generator.
"""
from . import inputs  # noqa: F401
from ._lib import (CODA_BF16, CODA_COL, CODA_F32, CODA_OP_BWD, CODA_OP_FWD,  # noqa: F401
                   CODA_OP_UNFUSED_BWD, CODA_OP_UNFUSED_FWD, CODA_ROW, CodaError, bwd, fwd, gemm, lib,
                   workspace, workspace_bytes)
