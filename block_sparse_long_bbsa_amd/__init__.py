"""BigBird block-sparse attention forward for AMD MI355X (gfx950).

The compute lives in the HIP library ``libbbsa.so`` (built in-tree by
``block_sparse_long_bbsa_amd.build``) behind the C ABI declared in
``include/bbsa.h``.  ``block_sparse_long_bbsa_amd.bbsa`` is a thin ctypes
binding with the same function names; torch only supplies device memory and
streams.  There is no CPU fallback: if the library is missing or the tensors
are not on the GPU the binding raises.
"""
from .bbsa import (  # noqa: F401
    BBSA_BF16, BBSA_F32, BBSA_OK, BBSA_OK_FULL_FALLBACK, BBSA_ERR_ARG, BBSA_ERR_SHAPE,
    BBSA_ERR_UNSUPPORTED, BBSA_ERR_HIP, BBSA_ERR_PLAN, BBSA_ERR_CAPTURE, BBSA_ERR_SCRATCH, BbsaError, lib,
    library_path, bbsa_forward_noalloc, bbsa_forward_ex, bbsa_attention_probs, bbsa_backward, BBSA_FLAG_PAD_TO_BLOCK, BBSA_FLAG_QUERY_KEY_MASK,
    bbsa_plan_rand_attn, bbsa_check_rand_attn, bbsa_plan_rand_attn_capped, bbsa_check_rand_attn_capped,
    bbsa_truncate_rand_attn, bbsa_forward, bbsa_status_string,
    bbsa_release_workspace, bbsa_version, bbsa_timing_enable, bbsa_timing_read, bbsa_work_map,
)
