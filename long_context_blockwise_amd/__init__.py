"""One device's share of ring attention on AMD Instinct MI355X (gfx950).

The compute path is ``libringattn.so``: hand-written HIP kernels behind the C
ABI of ``include/ring_attn.h``.  This package holds its sources (``csrc/``),
the in-tree build (``build.py``), a thin ctypes binding (``ring_attn.py``)
and seeded synthetic workload inputs (``inputs.py``).  Importing the package
does not load the library; the first call does, and fails loudly when the
library is missing.
"""
from .ring_attn import (  # noqa: F401
    EXPORTS,
    RA_BF16,
    RA_CHECK_DELAY_COMPUTE,
    RA_CHECK_DELAY_COPY,
    RA_CHECK_MAX_SPIN_US,
    RA_CHECK_POISON,
    RA_CHUNK_DIAG,
    RA_CHUNK_FULL,
    RA_CHUNK_SKIP,
    RA_ERR_HIP,
    RA_ERR_INVALID_ARG,
    RA_ERR_UNSUPPORTED,
    RA_ERR_WORKSPACE,
    RA_F32,
    RA_FLAG_ACCUMULATE,
    RA_FLAG_NO_SPLIT_KV,
    RA_FLAG_SPLIT_KV,
    RA_FLAG_STAGE,
    RA_FP8_E4M3,
    RA_KV_SCALE_BLOCK,
    RA_NOALLOC_SCRATCH_BYTES,
    RA_OK,
    RingAttnContext,
    RingAttnError,
    ring_attn_bwd,
    ring_attn_bwd_workspace_size,
    ring_attn_fwd,
    ring_attn_fwd_noalloc,
    ring_attn_last_error,
    ring_attn_merge,
    ring_attn_plan,
    ring_attn_ring_order,
    ring_attn_version,
    ring_attn_workspace_size,
)
