"""HIP graph capture of bbsa_forward.

A forward call is recorded once into a graph (torch's CUDAGraph on ROCm,
i.e. hipStreamBeginCapture on torch's capture stream) and replayed several
times with eager work and synchronisations in between.  The call enqueues
only kernel launches (no memsets, no allocation once the workspace exists),
so every replay must equal the eager call exactly; sampled rows are also
compared with the oracle.  Covered: rows merged in LDS (no workspace), rows
long enough to need the workspace and the merge kernel, and the fp32 path.
"""
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


@pytest.mark.parametrize("B,H,L,block,r,dtype", [
    (2, 4, 2048, 64, 3, "bf16"),    # full rows of up to four chunks: merged in LDS
    (1, 2, 8192, 64, 3, "bf16"),    # eight chunks per full row: workspace + merge kernel
    (1, 3, 4096, 128, 2, "bf16"),   # block 128
    (1, 2, 1024, 64, 3, "f32"),     # fp32 chunks + merge kernel
])
def test_graph_replay_matches_eager(B, H, L, block, r, dtype):
    announce(f"graph B{B} H{H} L{L} block{block} r{r} {dtype}")
    seed = 31
    inp = workloads.make_case(B, H, L, 64, seed, dtype=dtype, valid=[L - 100 * i for i in range(B)])
    nb = L // block
    cplan, oplan = plans(H, nb, r, seed)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q, k, v = (to_dev(inp[n], tdt) for n in ("q", "k", "v"))
    mask = to_dev(inp["mask"], torch.float32)
    ra = torch.from_numpy(cplan).cuda()

    # Eager call first, on the stream the capture will use: it sizes that
    # stream's library workspace, so the captured call allocates nothing.
    cap_stream = torch.cuda.Stream()
    cap_stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap_stream):
        eager_out, st = bbsa.bbsa_forward(q, k, v, mask, ra, block, r)
    assert st == bbsa.BBSA_OK
    torch.cuda.synchronize()
    eager = eager_out.float().cpu().numpy()

    out = torch.empty_like(q)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap_stream):
        _, st_cap = bbsa.bbsa_forward(q, k, v, mask, ra, block, r, out=out)
    assert st_cap == bbsa.BBSA_OK
    torch.cuda.synchronize()

    for rep in range(3):
        out.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        assert np.array_equal(got, eager), f"replay {rep} differs from the eager call"

    blocks = sample_blocks(nb)
    want = oracle.forward(inp["q"], inp["k"], inp["v"], inp["mask"], oplan, block, query_blocks=blocks)
    assert_close(gather_rows(got.astype(np.float64), blocks, block), want, dtype, "graph replay vs oracle")


@pytest.mark.parametrize("B,H,L,block,r,qk", [
    (2, 2, 4096, 64, 3, False),     # global rows and columns split: workspace partials + merge kernel
    (1, 2, 2048, 128, 2, True),     # block 128, query x key masking
])
def test_backward_graph_replay_matches_eager(B, H, L, block, r, qk):
    # The backward keeps its row terms and partials in the stream's library
    # workspace; after an eager call has sized it, a captured call allocates
    # nothing and every replay equals the eager call bit for bit.
    announce(f"backward graph B{B} H{H} L{L} block{block} r{r} qk={qk}")
    seed = 37
    inp = workloads.make_case(B, H, L, 64, seed, valid=[L - 300 * i for i in range(B)])
    nb = L // block
    cplan, _ = plans(H, nb, r, seed)
    q, k, v = (to_dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    mask = to_dev(inp["mask"], torch.float32)
    ra = torch.from_numpy(cplan).cuda()
    g = torch.Generator(device="cuda").manual_seed(seed)
    dout = torch.randn(q.shape, generator=g, device="cuda").to(torch.bfloat16)
    out, lse, st = bbsa.bbsa_forward_ex(q, k, v, mask, ra, block, r, return_lse=True, query_key_mask=qk)
    assert st == bbsa.BBSA_OK
    cap_stream = torch.cuda.Stream()
    cap_stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap_stream):
        eager = bbsa.bbsa_backward(q, k, v, out, dout, lse, mask, ra, block, r, query_key_mask=qk)
    assert eager[3] == bbsa.BBSA_OK
    torch.cuda.synchronize()
    eager = [t.float().cpu().numpy() for t in eager[:3]]

    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    delta = torch.empty_like(lse)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap_stream):
        st_cap = bbsa.bbsa_backward(q, k, v, out, dout, lse, mask, ra, block, r, dq=dq, dk=dk, dv=dv,
                                    delta=delta, query_key_mask=qk)[3]
    assert st_cap == bbsa.BBSA_OK
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (dq, dk, dv):
            t.fill_(float("nan"))    # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t, e in zip(("dq", "dk", "dv"), (dq, dk, dv), eager):
            assert np.array_equal(t.float().cpu().numpy(), e), f"replay {rep}: {name} differs from the eager call"


def _hip():
    import ctypes
    h = ctypes.CDLL("libamdhip64.so")
    h.hipStreamBeginCapture.argtypes = [ctypes.c_void_p, ctypes.c_int]
    h.hipStreamBeginCapture.restype = ctypes.c_int
    h.hipStreamEndCapture.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
    h.hipStreamEndCapture.restype = ctypes.c_int
    h.hipGraphDestroy.argtypes = [ctypes.c_void_p]
    h.hipGraphDestroy.restype = ctypes.c_int
    return h


def test_workspace_growth_during_capture_is_refused():
    # A stream that has never run a call needing the workspace is captured
    # (relaxed mode, HIP's own API): the call must return BBSA_ERR_CAPTURE
    # before touching the stream, and the capture must still end cleanly.
    import ctypes
    announce("capture without a sized workspace")
    inp = workloads.make_case(1, 2, 8192, 64, 33)
    plan = bbsa.bbsa_plan_rand_attn(2, 128, 3, 33)
    q, k, v = (to_dev(inp[n], torch.bfloat16) for n in ("q", "k", "v"))
    ra = torch.from_numpy(plan).cuda()
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    hip = _hip()
    HIP_CAPTURE_RELAXED = 2
    assert hip.hipStreamBeginCapture(ctypes.c_void_p(s.cuda_stream), HIP_CAPTURE_RELAXED) == 0
    st = bbsa.lib().bbsa_forward(q.data_ptr(), k.data_ptr(), v.data_ptr(), None, ra.data_ptr(),
                                 1, 2, 8192, 64, 64, 3, out.data_ptr(), ctypes.c_void_p(s.cuda_stream),
                                 bbsa.BBSA_BF16)
    graph = ctypes.c_void_p()
    assert hip.hipStreamEndCapture(ctypes.c_void_p(s.cuda_stream), ctypes.byref(graph)) == 0
    if graph.value:
        hip.hipGraphDestroy(graph)
    assert st == bbsa.BBSA_ERR_CAPTURE
    # The same stream works eagerly afterwards.
    with torch.cuda.stream(s):
        got, st2 = bbsa.bbsa_forward(q, k, v, None, ra, 64, 3)
    s.synchronize()
    assert st2 == bbsa.BBSA_OK
    blocks = sample_blocks(128)
    want = oracle.forward(inp["q"], inp["k"], inp["v"], None, plan, 64, query_blocks=blocks)
    assert_close(gather_rows(got.float().cpu().numpy().astype(np.float64), blocks, 64), want, "bf16",
                 "eager after refused capture")
