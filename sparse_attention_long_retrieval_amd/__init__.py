"""MI355X (gfx950) head-wise sparse attention step of RTPurbo.

The compute path is librtp.so (hand-written HIP kernels behind the C ABI in
include/rtp.h); this package only binds it.  Build with
`python -m sparse_attention_long_retrieval_amd.build`.
"""
from .binding import (  # noqa: F401
    OP_APPEND, OP_CLUSTER_BUILD, OP_CLUSTER_DECODE, OP_DECODE, OP_DECODE_STEP, OP_PREFILL, OP_SWA,
    EXPORTED,
    LIB_PATH, Debug, Layer, RtpError, cluster_build, decode_cluster_attn, decode_sparse_attn,
    decode_sparse_attn_noalloc, decode_step,
    decode_topk, index_append, lib, prefill_chunk, ring_append, swa_attn, swa_attn_ring,
    workspace_size,
)
