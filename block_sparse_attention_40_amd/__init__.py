"""MoBA (Mixture of Block Attention) prefill forward for AMD MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
include/moba.h (libmoba.so, built in-tree); this package is a thin binding.
"""
from ._lib import (  # noqa: F401
    DTYPE_BF16,
    DECODE_CHUNK,
    DTYPE_F32,
    GATE_KINDS,
    LIB_PATH,
    MAX_DECODE_GROUP,
    MAX_DECODE_TOPK,
    MobaError,
    decode_workspace_bytes,
    moba_decode_fwd,
    moba_decode_means,
    bwd_workspace_bytes,
    moba_attn_bwd,
    moba_attn_fwd,
    moba_attn_fwd_noalloc,
    NOALLOC_SCRATCH_BYTES,
    moba_attn_fwd_train,
    moba_gate,
    moba_meanpool,
    moba_minmaxpool,
    plan_chunk_blocks,
    plan_info,
    profile_enable,
    profile_read,
    STAGES,
    status_string,
    version,
    workspace_bytes,
)
