"""C ABI surface checks that need no GPU.

The library loads, exports every function declared in include/bbsa.h, and
rejects invalid forward arguments with the documented status codes.  Every
forward call here is invalid, so it returns before any HIP call.
"""
import ctypes
import os
import re

import pytest

bbsa = pytest.importorskip("block_sparse_long_bbsa_amd.bbsa")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    try:
        return bbsa.lib()
    except RuntimeError as e:
        pytest.skip(str(e))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "bbsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(bbsa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("bbsa_plan_rand_attn", "bbsa_check_rand_attn", "bbsa_forward",
                     "bbsa_status_string", "bbsa_release_workspace"):
        assert required in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in (0, 1, -1, -2, -3, -4, -5, -6, -7):
        assert bbsa.bbsa_status_string(code) and bbsa.bbsa_status_string(code) != "unknown status"
    assert bbsa.bbsa_status_string(42) == "unknown status"
    assert bbsa.bbsa_version() >= 100


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def call(lib, B=1, H=1, L=1024, d=64, block=64, r=3, dtype=0, q=FAKE, k=FAKE, v=FAKE,
         out=FAKE, ra=FAKE, mask=None):
    return lib.bbsa_forward(q, k, v, mask, ra, B, H, L, d, block, r, out, None, dtype)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(k=None), -1), (dict(v=None), -1), (dict(out=None), -1),
    (dict(B=0), -1), (dict(H=-1), -1), (dict(L=0), -1), (dict(d=0), -1), (dict(block=0), -1),
    (dict(r=0), -1), (dict(r=-2), -1),
    (dict(ra=None), -1),                       # sparse path needs the plan
    (dict(L=1000), -2), (dict(L=1024 + 64, block=128), -2),
    (dict(d=128), -3), (dict(block=32, L=1024), -3), (dict(dtype=7), -3),
    (dict(B=1 << 20, H=1 << 10, L=1 << 14), -3),   # beyond the supported size
    (dict(L=8192, r=60), -3),                  # a middle row would list 65 key blocks
    (dict(q=ctypes.c_void_p(0x1008)), -1),     # device pointers must be 16-byte aligned
    (dict(out=ctypes.c_void_p(0x1004)), -1),
    (dict(mask=ctypes.c_void_p(0x1008)), -1),
    (dict(ra=ctypes.c_void_p(0x1002)), -1),    # the plan 4-byte aligned
])
def test_forward_rejects_invalid_arguments(lib, kw, code):
    assert call(lib, **kw) == code


def test_noalloc_validates_like_forward(lib):
    # Same argument checks as bbsa_forward; a call whose partials would not fit
    # the fixed scratch is refused with its own status.  No HIP call happens.
    for kw, code in [(dict(q=None), -1), (dict(L=1000), -2), (dict(d=128), -3), (dict(ra=None), -1)]:
        args = dict(B=1, H=1, L=1024, d=64, block=64, r=3, dtype=0, q=FAKE, k=FAKE, v=FAKE, out=FAKE, ra=FAKE,
                    mask=None)
        args.update(kw)
        st = lib.bbsa_forward_noalloc(args["q"], args["k"], args["v"], args["mask"], args["ra"], args["B"],
                                      args["H"], args["L"], args["d"], args["block"], args["r"], args["out"],
                                      None, args["dtype"])
        assert st == code
    st = lib.bbsa_forward_noalloc(FAKE, FAKE, FAKE, None, FAKE, 64, 16, 32768, 64, 64, 3, FAKE, None, 0)
    assert st == bbsa.BBSA_ERR_SCRATCH


def test_forward_ex_validates(lib):
    # Unknown flag bits, a ragged length without the padding flag, and the
    # usual argument errors; no HIP call happens for any of them.
    def ex(L=1024, flags=0, lse=None, q=FAKE):
        return lib.bbsa_forward_ex(q, FAKE, FAKE, None, FAKE, 1, 1, L, 64, 64, 3, FAKE, lse, None, 0, flags)
    assert ex(flags=8) == bbsa.BBSA_ERR_ARG
    assert ex(flags=0x80000000) == bbsa.BBSA_ERR_ARG
    assert ex(L=1000) == bbsa.BBSA_ERR_SHAPE
    assert ex(q=None) == bbsa.BBSA_ERR_ARG
    assert ex(L=1000, flags=1, lse=ctypes.c_void_p(0x1002)) == bbsa.BBSA_ERR_ARG   # lse 4-byte aligned
