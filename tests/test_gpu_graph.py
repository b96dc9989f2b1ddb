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

    # Eager call first: it also sizes the library workspace, so the captured
    # call allocates nothing.
    eager_out, st = bbsa.bbsa_forward(q, k, v, mask, ra, block, r)
    assert st == bbsa.BBSA_OK
    torch.cuda.synchronize()
    eager = eager_out.float().cpu().numpy()

    out = torch.empty_like(q)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
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
