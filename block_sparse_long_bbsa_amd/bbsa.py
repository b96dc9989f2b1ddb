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
        L.bbsa_forward.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int] * 6 + \
            [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        L.bbsa_forward.restype = ctypes.c_int
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


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BBSA_BF16
    if t.dtype == torch.float32:
        return BBSA_F32
    raise ValueError(f"unsupported dtype {t.dtype}")


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
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_cuda or not out.is_contiguous():
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
        if L % block == 0 and tuple(rand_attn.shape) != (H, L // block - 2, r):
            raise ValueError(f"rand_attn must be [H, nb-2, r] = {(H, L // block - 2, r)}")
        rptr = rand_attn.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = lib().bbsa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), mptr, rptr,
                                B, H, L, d, int(block), int(r), out.data_ptr(),
                                ctypes.c_void_p(handle), code)
    if st < 0:
        if st == BBSA_ERR_HIP:
            raise BbsaError(st, "bbsa_forward")
        raise ValueError(f"bbsa_forward: status {st}: {bbsa_status_string(st)}")
    if st == BBSA_OK_FULL_FALLBACK and warn_fallback:
        warnings.warn(f"sequence length {L} <= (5 + 2*{r}) * {block}: computed full attention")
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
