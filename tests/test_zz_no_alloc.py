"""bbsa_forward_noalloc: the forward for callers that cannot allocate.

Called through the C ABI, it must give exactly what bbsa_forward gives on the
same inputs (same kernels; only the split-K scratch differs), and match the
oracle within the stated tolerances, on two calls in a row where the second
is smaller (the fixed scratch array keeps the first call's contents, which
the second must not depend on).  A call that would need more scratch than
the fixed maximum is refused before any HIP call.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from block_sparse_long_bbsa_amd import bbsa, workloads
from gpu_helpers import announce, assert_close, gather_rows, plans, sample_blocks, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bbsa.lib()


def _inputs(B, H, L, block, r, dtype, seed, valid):
    inp = workloads.make_case(B, H, L, 64, seed, dtype=dtype, valid=valid)
    cplan, oplan = plans(H, L // block, r, seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    dev = {n: to_dev(inp[n], tdt) for n in ("q", "k", "v")}
    dev["mask"] = to_dev(inp["mask"], torch.float32)
    dev["ra"] = torch.from_numpy(cplan).cuda()
    return inp, oplan, dev


def _both(dev, block, r, stream=None):
    want, st = bbsa.bbsa_forward(dev["q"], dev["k"], dev["v"], dev["mask"], dev["ra"], block, r, stream=stream)
    out = torch.full_like(dev["q"], float("nan"))
    got, st2 = bbsa.bbsa_forward_noalloc(dev["q"], dev["k"], dev["v"], dev["mask"], dev["ra"], block, r, out,
                                         stream=stream)
    torch.cuda.synchronize()
    assert st == st2 == bbsa.BBSA_OK
    return got, want


@pytest.mark.parametrize("first,second", [
    # (B, H, L, block, r, dtype, seed, valid): both calls need split-K scratch.
    ((1, 4, 16384, 64, 3, "bf16", 61, (16000,)), (1, 2, 8192, 64, 3, "bf16", 62, (8000,))),
    ((1, 3, 16384, 128, 2, "bf16", 63, None), (1, 2, 5120, 128, 2, "bf16", 64, (5000,))),
    ((1, 2, 2048, 64, 3, "f32", 65, (1900,)), (1, 1, 1024, 64, 3, "f32", 66, None)),
])
def test_noalloc_matches_forward_on_two_calls(first, second):
    for case in (first, second):
        B, H, L, block, r, dtype, seed, valid = case
        announce(f"noalloc B{B} H{H} L{L} block{block} r{r} {dtype}")
        inp, oplan, dev = _inputs(B, H, L, block, r, dtype, seed, valid)
        got, want = _both(dev, block, r)
        assert torch.equal(got, want), "noalloc output differs from bbsa_forward"
        nb = L // block
        blocks = sample_blocks(nb) if L > 4096 else list(range(nb))
        ref = oracle.forward(inp["q"], inp["k"], inp["v"], inp["mask"], oplan, block, query_blocks=blocks)
        assert_close(gather_rows(got.float().cpu().numpy().astype(np.float64), blocks, block), ref, dtype,
                     f"noalloc L{L} {dtype}")


def test_noalloc_on_a_side_stream():
    announce("noalloc side stream")
    inp, oplan, dev = _inputs(1, 2, 8192, 64, 3, "bf16", 67, (7000,))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        got, want = _both(dev, 64, 3, stream=s)
    assert torch.equal(got, want)


def test_noalloc_refuses_more_than_its_scratch():
    # 64 x 16 pairs of 32768-token rows: even with the longest full-row chunks
    # (4096 keys, 4 per partial) the two global row tiles of each pair need
    # 2 * ceil(32768 / 16384) partials, 4096 in all (> 1007), so the call is
    # refused during validation, before any HIP call; the pointers are never
    # used.  The count is checked here first: a shape that fitted would launch
    # kernels on the fake pointers.
    B, H, L, block = 64, 16, 32768, 64
    assert B * H * 2 * (block // 64) * -(-L // (4 * 4096)) > 1007
    fake = ctypes.c_void_p(0x10000)
    st = bbsa.lib().bbsa_forward_noalloc(fake, fake, fake, None, fake, B, H, L, 64, block, 3, fake, None,
                                         bbsa.BBSA_BF16)
    assert st == bbsa.BBSA_ERR_SCRATCH
