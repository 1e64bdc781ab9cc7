"""TiDAR decode-step hot path for MI355X (gfx950): Python binding of libtidar.

The compute runs in the HIP library ``libtidar.so`` (C ABI in
``include/tidar.h``); this package only marshals torch tensors into it.
Importing it without the built library raises ImportError.
"""
from ._lib import (  # noqa: F401
    AttnDesc, TidarError, attn_step, attn_workspace, attn_workspace_bytes, kv_commit, last_error, load,
    make_attn_desc, reject_sample, reject_sample_noalloc, reject_workspace_bytes, token_logprobs, logprob_workspace_bytes,
    DTYPE_BF16, DTYPE_F32, EXPORTS, LIB_PATH, ceiling, attn_stamps,
)
from .step import DecodeStep  # noqa: F401

__all__ = [
    "AttnDesc", "TidarError", "attn_step", "attn_workspace", "attn_workspace_bytes", "kv_commit", "last_error",
    "make_attn_desc", "reject_sample", "reject_sample_noalloc", "reject_workspace_bytes", "token_logprobs", "logprob_workspace_bytes",
    "DecodeStep", "DTYPE_BF16",
    "DTYPE_F32", "EXPORTS", "LIB_PATH",
]
