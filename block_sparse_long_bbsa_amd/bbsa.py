"""ctypes binding of ``libbbsa.so`` (argument marshalling only).

Every function mirrors the C entry point of the same name in
``include/bbsa.h``.  Tensors must be contiguous torch tensors in GPU memory;
``bbsa_forward`` enqueues the kernels on torch's current stream of the
tensors' device.
"""
from __future__ import annotations

import ctypes
import os
import warnings

import numpy as np

BBSA_BF16 = 0
BBSA_F32 = 1

BBSA_OK = 0
BBSA_OK_FULL_FALLBACK = 1
BBSA_ERR_ARG = -1
BBSA_ERR_SHAPE = -2
BBSA_ERR_UNSUPPORTED = -3
BBSA_ERR_HIP = -4
BBSA_ERR_PLAN = -5
BBSA_ERR_CAPTURE = -6
BBSA_ERR_SCRATCH = -7

BBSA_FLAG_PAD_TO_BLOCK = 1
BBSA_FLAG_QUERY_KEY_MASK = 2
BBSA_FLAG_KEEP_PADDED_BLOCKS = 4

WORK_RECORD_INTS = 80

_LIB = None


class BbsaError(RuntimeError):
    """A negative status from the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {bbsa_status_string(status)}")


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbbsa.so")


def lib() -> ctypes.CDLL:
    """Load ``libbbsa.so`` once; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m block_sparse_long_bbsa_amd.build`")
        L = ctypes.CDLL(path)
        i32p = ctypes.POINTER(ctypes.c_int32)
        L.bbsa_plan_rand_attn.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64]
        L.bbsa_plan_rand_attn.restype = ctypes.c_int
        L.bbsa_check_rand_attn.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        L.bbsa_check_rand_attn.restype = ctypes.c_int
        L.bbsa_plan_rand_attn_capped.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                                 ctypes.c_int, ctypes.c_int]
        L.bbsa_plan_rand_attn_capped.restype = ctypes.c_int
        L.bbsa_check_rand_attn_capped.argtypes = [i32p] + [ctypes.c_int] * 5
        L.bbsa_check_rand_attn_capped.restype = ctypes.c_int
        L.bbsa_truncate_rand_attn.argtypes = [i32p, ctypes.c_int, ctypes.c_int, ctypes.c_int, i32p, ctypes.c_int]
        L.bbsa_truncate_rand_attn.restype = ctypes.c_int
        L.bbsa_forward.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + \
            [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        L.bbsa_forward.restype = ctypes.c_int
        L.bbsa_forward_noalloc.argtypes = L.bbsa_forward.argtypes
        L.bbsa_forward_noalloc.restype = ctypes.c_int
        L.bbsa_forward_ex.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + \
            [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_uint]
        L.bbsa_forward_ex.restype = ctypes.c_int
        L.bbsa_attention_probs.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int] * 6 + \
            [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_uint]
        L.bbsa_attention_probs.restype = ctypes.c_int
        L.bbsa_backward.argtypes = [ctypes.c_void_p] * 8 + [ctypes.c_int] * 6 + [ctypes.c_void_p] * 5 + \
            [ctypes.c_int, ctypes.c_uint]
        L.bbsa_backward.restype = ctypes.c_int
        L.bbsa_status_string.argtypes = [ctypes.c_int]
        L.bbsa_status_string.restype = ctypes.c_char_p
        L.bbsa_release_workspace.argtypes = []
        L.bbsa_release_workspace.restype = None
        L.bbsa_version.argtypes = []
        L.bbsa_version.restype = ctypes.c_int
        L.bbsa_timing_enable.argtypes = [ctypes.c_int]
        L.bbsa_timing_enable.restype = ctypes.c_int
        dp = ctypes.POINTER(ctypes.c_double)
        L.bbsa_timing_read.argtypes = [dp, dp, ctypes.POINTER(ctypes.c_int)]
        L.bbsa_timing_read.restype = ctypes.c_int
        i64p = ctypes.POINTER(ctypes.c_int64)
        L.bbsa_work_map.argtypes = [ctypes.c_int] * 7 + [ctypes.c_uint, i32p, i32p, ctypes.c_int64, i64p, i64p]
        L.bbsa_work_map.restype = ctypes.c_int
        _LIB = L
    return _LIB


def bbsa_status_string(status: int) -> str:
    return lib().bbsa_status_string(int(status)).decode()


def bbsa_version() -> int:
    return lib().bbsa_version()


def bbsa_plan_rand_attn(H: int, nb: int, r: int, seed: int) -> np.ndarray:
    """Host plan as int32 ``[H, nb-2, r]`` (see include/bbsa.h)."""
    n = max(H, 0) * max(nb - 2, 0) * max(r, 0)
    buf = np.zeros(max(n, 1), dtype=np.int32)
    st = lib().bbsa_plan_rand_attn(buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   int(H), int(nb), int(r), ctypes.c_uint64(int(seed) & (2**64 - 1)))
    if st < 0:
        raise BbsaError(st, "bbsa_plan_rand_attn")
    return buf[:n].reshape(H, nb - 2, r)


def bbsa_check_rand_attn(rand_attn: np.ndarray, nb: int, r: int) -> int:
    """Status of the host plan check (BBSA_OK or BBSA_ERR_PLAN, ...)."""
    ra = np.ascontiguousarray(rand_attn, dtype=np.int32)
    H = ra.shape[0] if ra.ndim == 3 else 0
    if ra.ndim != 3 or ra.shape[1] != nb - 2 or ra.shape[2] != r:
        return BBSA_ERR_SHAPE
    return lib().bbsa_check_rand_attn(ra.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), H, int(nb), int(r))


def bbsa_plan_rand_attn_capped(H: int, nb: int, r: int, seed: int, block: int, last_idx: int) -> np.ndarray:
    """Host plan with the random range capped to the first ``last_idx``
    tokens (see include/bbsa.h)."""
    n = max(H, 0) * max(nb - 2, 0) * max(r, 0)
    buf = np.zeros(max(n, 1), dtype=np.int32)
    st = lib().bbsa_plan_rand_attn_capped(buf.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(H), int(nb),
                                          int(r), ctypes.c_uint64(int(seed) & (2**64 - 1)), int(block),
                                          int(last_idx))
    if st < 0:
        raise BbsaError(st, "bbsa_plan_rand_attn_capped")
    return buf[:n].reshape(H, nb - 2, r)


def bbsa_check_rand_attn_capped(rand_attn: np.ndarray, nb: int, r: int, block: int, last_idx: int) -> int:
    ra = np.ascontiguousarray(rand_attn, dtype=np.int32)
    if ra.ndim != 3 or ra.shape[1] != nb - 2 or ra.shape[2] != r:
        return BBSA_ERR_SHAPE
    return lib().bbsa_check_rand_attn_capped(ra.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), ra.shape[0],
                                             int(nb), int(r), int(block), int(last_idx))


def bbsa_truncate_rand_attn(rand_attn: np.ndarray, nb: int):
    """Returns ``(status, plan)``: the first nb-2 rows of a longer plan."""
    src = np.ascontiguousarray(rand_attn, dtype=np.int32)
    H, rows, r = src.shape
    dst = np.zeros((H, max(nb - 2, 1), r), dtype=np.int32)
    i32p = ctypes.POINTER(ctypes.c_int32)
    st = lib().bbsa_truncate_rand_attn(src.ctypes.data_as(i32p), H, rows + 2, r, dst.ctypes.data_as(i32p), int(nb))
    return st, dst[:, :max(nb - 2, 0)]


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BBSA_BF16
    if t.dtype == torch.float32:
        return BBSA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


def _marshal(q, k, v, mask, rand_attn, block, r, out, stream, pad=False):
    """Check the tensors and return the C arguments of a forward call."""
    import torch
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must share one [B, H, L, d] shape")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype")
    B, H, L, d = q.shape
    code = _dtype_code(q)
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_cuda or not out.is_contiguous():
        raise ValueError("out must be a contiguous GPU tensor shaped and typed like q")
    mptr = None
    if mask is not None:
        if not mask.is_cuda or mask.dtype != torch.float32 or tuple(mask.shape) != (B, L) \
                or not mask.is_contiguous():
            raise ValueError("mask must be a contiguous float32 [B, L] GPU tensor")
        mptr = mask.data_ptr()
    rptr = None
    if rand_attn is not None:
        if not rand_attn.is_cuda or rand_attn.dtype != torch.int32 or not rand_attn.is_contiguous():
            raise ValueError("rand_attn must be a contiguous int32 GPU tensor")
        nb = -(-L // block)
        if tuple(rand_attn.shape) != (H, nb - 2, r) and (L % block == 0 or pad):
            raise ValueError(f"rand_attn must be [H, nb-2, r] = {(H, nb - 2, r)}")
        rptr = rand_attn.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    return (q.data_ptr(), k.data_ptr(), v.data_ptr(), mptr, rptr, B, H, L, d, int(block), int(r),
            out.data_ptr(), ctypes.c_void_p(handle), code)


def _status(st, where, L, block, r, warn_fallback):
    if st < 0:
        if st in (BBSA_ERR_HIP, BBSA_ERR_CAPTURE, BBSA_ERR_SCRATCH):
            raise BbsaError(st, where)
        raise ValueError(f"{where}: status {st}: {bbsa_status_string(st)}")
    if st == BBSA_OK_FULL_FALLBACK and warn_fallback:
        warnings.warn(f"sequence length {L} <= (5 + 2*{r}) * {block}: computed full attention")


def bbsa_forward(q, k, v, mask, rand_attn, block: int, r: int, out=None, stream=None,
                 warn_fallback: bool = True):
    """Block-sparse attention forward on the GPU.

    q, k, v: contiguous ``[B, H, L, d]`` bf16 or fp32 GPU tensors.
    mask: float32 ``[B, L]`` GPU tensor or None.  rand_attn: int32
    ``[H, nb-2, r]`` GPU tensor (may be None when L <= (5+2r)*block).
    Returns ``(out, status)``; status 1 means full attention was computed
    (a warning is issued, as the reference layer does).
    """
    import torch
    if out is None:
        out = torch.empty_like(q)
    args = _marshal(q, k, v, mask, rand_attn, block, r, out, stream)
    with torch.cuda.device(q.device):
        st = lib().bbsa_forward(*args)
    _status(st, "bbsa_forward", q.shape[2], block, r, warn_fallback)
    return out, st


def bbsa_forward_ex(q, k, v, mask, rand_attn, block: int, r: int, out=None, lse=None, stream=None,
                    pad_to_block: bool = False, query_key_mask: bool = False, return_lse: bool = False,
                    warn_fallback: bool = True, keep_padded_blocks: bool = False):
    """``bbsa_forward`` with options (see include/bbsa.h):

    pad_to_block: L need not be a multiple of ``block`` (the sequence is
    handled as padded to ceil(L/block) blocks; rand_attn is the plan of that
    block count).  query_key_mask: bias -10000 (1 - m[query] m[key]).
    keep_padded_blocks: also compute key blocks whose keys all have mask 0
    (by default a tile that attends a key of mask 1 leaves them out, which
    does not change the result).  return_lse / lse: also produce the float32
    ``[B, H, L]`` row log-sum-exp.  Returns ``(out, status)`` or
    ``(out, lse, status)``.
    """
    import torch
    if out is None:
        out = torch.empty_like(q)
    B, H, L, _ = q.shape
    if lse is None and return_lse:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    if lse is not None:
        if not lse.is_cuda or lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, L) or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [B, H, L] GPU tensor")
    args = list(_marshal(q, k, v, mask, rand_attn, block, r, out, stream, pad=pad_to_block))
    flags = (BBSA_FLAG_PAD_TO_BLOCK if pad_to_block else 0) | (BBSA_FLAG_QUERY_KEY_MASK if query_key_mask else 0) | \
        (BBSA_FLAG_KEEP_PADDED_BLOCKS if keep_padded_blocks else 0)
    cargs = args[:12] + [None if lse is None else lse.data_ptr(), args[12], args[13], flags]
    with torch.cuda.device(q.device):
        st = lib().bbsa_forward_ex(*cargs)
    _status(st, "bbsa_forward_ex", L, block, r, warn_fallback)
    return (out, lse, st) if lse is not None else (out, st)


def bbsa_attention_probs(q, k, mask, rand_attn, block: int, r: int, probs=None, stream=None,
                         pad_to_block: bool = False, query_key_mask: bool = False):
    """Dense float32 ``[B, H, L, L]`` attention probabilities of the pattern
    (zeros outside it); see include/bbsa.h.  Returns ``(probs, status)``."""
    import torch
    B, H, L, d = q.shape
    if probs is None:
        probs = torch.empty((B, H, L, L), dtype=torch.float32, device=q.device)
    if not probs.is_cuda or probs.dtype != torch.float32 or tuple(probs.shape) != (B, H, L, L) \
            or not probs.is_contiguous():
        raise ValueError("probs must be a contiguous float32 [B, H, L, L] GPU tensor")
    args = _marshal(q, k, q, mask, rand_attn, block, r, q, stream, pad=pad_to_block)
    flags = (BBSA_FLAG_PAD_TO_BLOCK if pad_to_block else 0) | (BBSA_FLAG_QUERY_KEY_MASK if query_key_mask else 0)
    # (q, k, mask, rand_attn, B, H, L, d, block, r, probs, stream, dtype, flags)
    cargs = [args[0], args[1], args[3], args[4]] + list(args[5:11]) + [probs.data_ptr(), args[12], args[13], flags]
    with torch.cuda.device(q.device):
        st = lib().bbsa_attention_probs(*cargs)
    _status(st, "bbsa_attention_probs", L, block, r, False)
    return probs, st


def bbsa_backward(q, k, v, out, dout, lse, mask, rand_attn, block: int, r: int, dq=None, dk=None, dv=None,
                  delta=None, stream=None, pad_to_block: bool = False, query_key_mask: bool = False,
                  keep_padded_blocks: bool = False):
    """Gradients (dq, dk, dv) of the forward's output; ``out`` and ``lse``
    come from ``bbsa_forward_ex`` with the same arguments (see
    include/bbsa.h).  keep_padded_blocks: also compute the steps whose keys
    all have mask 0 (left out by default where they add nothing).
    Returns ``(dq, dk, dv, status)``."""
    import torch
    B, H, L, d = q.shape
    for t in (out, dout):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError("out and dout must be contiguous GPU tensors shaped and typed like q")
    if not lse.is_cuda or lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, L) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B, H, L] GPU tensor")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t in (dq, dk, dv):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_cuda or not t.is_contiguous():
            raise ValueError("dq, dk, dv must be contiguous GPU tensors shaped and typed like q")
    if delta is None:
        delta = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    args = _marshal(q, k, v, mask, rand_attn, block, r, out, stream, pad=pad_to_block)
    flags = (BBSA_FLAG_PAD_TO_BLOCK if pad_to_block else 0) | (BBSA_FLAG_QUERY_KEY_MASK if query_key_mask else 0) | \
        (BBSA_FLAG_KEEP_PADDED_BLOCKS if keep_padded_blocks else 0)
    cargs = [args[0], args[1], args[2], out.data_ptr(), dout.data_ptr(), lse.data_ptr(), args[3], args[4]] + \
        list(args[5:11]) + [dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(), args[12], args[13], flags]
    with torch.cuda.device(q.device):
        st = lib().bbsa_backward(*cargs)
    _status(st, "bbsa_backward", L, block, r, False)
    return dq, dk, dv, st


def bbsa_forward_noalloc(q, k, v, mask, rand_attn, block: int, r: int, out, stream=None,
                         warn_fallback: bool = True):
    """``bbsa_forward`` through the entry point that allocates nothing (the
    library's fixed per-device scratch; see include/bbsa.h).  ``out`` must be
    given.  Returns ``(out, status)``."""
    import torch
    if out is None:
        raise ValueError("bbsa_forward_noalloc needs an output tensor")
    args = _marshal(q, k, v, mask, rand_attn, block, r, out, stream)
    with torch.cuda.device(q.device):
        st = lib().bbsa_forward_noalloc(*args)
    _status(st, "bbsa_forward_noalloc", q.shape[2], block, r, warn_fallback)
    return out, st


def bbsa_release_workspace() -> None:
    lib().bbsa_release_workspace()


def bbsa_timing_enable(enable: bool) -> None:
    st = lib().bbsa_timing_enable(1 if enable else 0)
    if st < 0:
        raise BbsaError(st, "bbsa_timing_enable")


def bbsa_timing_read():
    """Returns (main_kernel_ms_total, combine_kernel_ms_total, calls)."""
    a, c, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int()
    st = lib().bbsa_timing_read(ctypes.byref(a), ctypes.byref(c), ctypes.byref(n))
    if st < 0:
        raise BbsaError(st, "bbsa_timing_read")
    return a.value, c.value, n.value


def bbsa_work_map(B: int, H: int, L: int, d: int, block: int, r: int, dtype: int, rand_attn=None,
                  flags: int = 0):
    """The attention kernel's work decomposition for a call's shape (see
    ``bbsa_work_map`` in include/bbsa.h): returns ``(status, grid, records)``
    with ``records`` an int32 array ``[units, 80]``."""
    i32p = ctypes.POINTER(ctypes.c_int32)
    ra = None
    rptr = None
    if rand_attn is not None:
        ra = np.ascontiguousarray(rand_attn, dtype=np.int32)
        rptr = ra.ctypes.data_as(i32p)
    count, grid = ctypes.c_int64(), ctypes.c_int64()
    st = lib().bbsa_work_map(B, H, L, d, block, r, dtype, flags, rptr, None, 0, ctypes.byref(count),
                             ctypes.byref(grid))
    if st < 0:
        return st, 0, np.zeros((0, WORK_RECORD_INTS), dtype=np.int32)
    rec = np.zeros((max(count.value, 1), WORK_RECORD_INTS), dtype=np.int32)
    st = lib().bbsa_work_map(B, H, L, d, block, r, dtype, flags, rptr, rec.ctypes.data_as(i32p), count.value,
                             ctypes.byref(count), ctypes.byref(grid))
    return st, grid.value, rec[:count.value]
