"""The path captured in a HIP graph: pack A, pack B and the multiply-accumulate
(plain, split-K with its reduce, and the alpha/beta form) recorded once and
replayed several times, with eager work and synchronisations between the
replays; every replay must equal the eager result bit for bit. The library's
kernels use no memset and allocate nothing, so they are capturable as they
are."""
import numpy as np
import pytest
import torch

import bf16_matrix_multiply_amd as bmm
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("form", ["plain_tiled", "plain_tiled128", "plain_direct", "splitk", "scaled",
                                  "k8"])
def test_graph_replays_match_eager(form):
    w = workloads.custom(1, 528, 520, 1040, "bf16", c_tensor=True)
    inp = workloads.make_inputs(w, seed=6)
    a, b = gu.dev_u16(inp["a"]), gu.dev_u16(inp["b"])
    C = torch.from_numpy(inp["c_tensor"]).cuda()
    ka = 8 if form == "k8" else 16
    A = torch.empty((1, w.M_rep, w.K // ka, 16, ka // 2), dtype=torch.int32, device="cuda")
    B = torch.empty((1, w.N_rep, w.K // ka, 8, ka // 2), dtype=torch.int32, device="cuda")
    D = torch.empty((1, w.M_rep, w.N_rep, 16, 8), dtype=torch.float32, device="cuda")
    splits = 4
    ws = torch.empty(bmm.splitk_workspace_bytes(1, w.M_rep, w.N_rep, w.K // 16, 16, splits) // 4,
                     dtype=torch.float32, device="cuda")
    pack_kw = {} if ka == 16 else {"atom_k": 8}

    def step():
        bmm.pack_operand(a, 16, out=A, **pack_kw)
        bmm.pack_operand(b, 8, out=B, **pack_kw)
        if form == "splitk":
            bmm.mma_tile_splitk(A, B, C, 0.0, "bf16", splits, out=D, workspace=ws)
        elif form == "scaled":
            bmm.mma_tile(A, B, C, 0.0, "bf16", out=D, kernel="tiled", alpha=0.5, beta=-1.5)
        elif form == "plain_direct":
            bmm.mma_tile(A, B, C, 0.0, "bf16", out=D, kernel="direct")
        elif form == "plain_tiled128":
            bmm.mma_tile(A, B, C, 0.0, "bf16", out=D, kernel="tiled128")
        else:
            bmm.mma_tile(A, B, C, 0.0, "bf16", out=D, kernel="tiled")

    step()
    torch.cuda.synchronize()
    eager = D.clone()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                       # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        D.fill_(float("nan"))
        A.zero_()
        B.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(D, eager), f"{form}: replay {i} differs from the eager result"
        # eager work between replays
        bmm.mma_tile(A, B, None, 1.0, "bf16", out=torch.empty_like(D), kernel="direct")
        torch.cuda.synchronize()
    assert not torch.isnan(D).any()
