"""The no-allocation split-K entry point (bmm_mma_tile_splitk_noalloc),
called through the C ABI: its result equals the workspace form's
(bmm_mma_tile_splitk with the same split count; same kernels, so the same
bits) on two calls in a row, the second with a smaller input, and on a third
call on the null stream; the results also meet the oracle's split-K bound.
A request beyond the static scratch is refused without touching D."""
import ctypes

import numpy as np
import pytest
import torch

import bf16_matrix_multiply_amd as bmm
import oracle
import workloads
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

ERANGE = -4


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(L, D, A, B, C, c, w, splits, null_stream=False):
    stream = None if null_stream else ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return L.bmm_mma_tile_splitk_noalloc(_ptr(D), _ptr(A), _ptr(B), _ptr(C), float(c), w.batch,
                                         w.M_rep, w.N_rep, w.K_rep, 1, 16, splits, stream)


# (workload, splits): the first uses the whole scratch (16 partials of 4 MiB),
# the second a smaller one, with a scalar C and ragged tiles.
CASES = [
    (workloads.custom(1, 1024, 1024, 8192, "bf16", "normal", "normal", c_tensor=True,
                      name="noalloc_full_scratch"), 16),
    (workloads.custom(1, 272, 520, 2080, "bf16", "normal", "normal", c_tensor=False,
                      name="noalloc_small_ragged"), 3),
]


def test_noalloc_equals_workspace_form_on_consecutive_calls():
    L = bmm.lib()
    results = []
    for w, splits in CASES:
        print(f"[noalloc] {w.name}: {w.M}x{w.N}x{w.K} splits={splits}", flush=True)
        need = bmm.splitk_workspace_bytes(w.batch, w.M_rep, w.N_rep, w.K_rep, 16, splits)
        assert need <= bmm.NOALLOC_SCRATCH_BYTES
        inp = workloads.make_inputs(w, seed=21)
        A = bmm.pack_operand(gu.dev_u16(inp["a"]), 16)
        B = bmm.pack_operand(gu.dev_u16(inp["b"]), 8)
        C = None if inp["c_tensor"] is None else torch.from_numpy(inp["c_tensor"]).cuda()
        c = float(inp["c_scalar"])
        shape = (w.batch, w.M_rep, w.N_rep, 16, 8)
        D = torch.full(shape, float("nan"), device="cuda")
        assert _noalloc(L, D, A, B, C, c, w, splits) == 0, L.bmm_last_error().decode()
        ws = torch.empty(max(need // 4, 1), dtype=torch.float32, device="cuda")
        Dw = torch.full(shape, float("nan"), device="cuda")
        bmm.mma_tile_splitk(A, B, C, c, w.dtype, splits, out=Dw, workspace=ws)
        torch.cuda.synchronize()
        got, ref = D.cpu().numpy(), Dw.cpu().numpy()
        assert not np.isnan(got).any(), f"{w.name}: unwritten outputs"
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), w.name
        results.append((w, inp, got, splits))
        last = (A, B, C, c, shape)
    # A third call on the null stream (the scratch of the current device), the
    # smaller input again: the same bits.
    A, B, C, c, shape = last
    w, _, got_prev, splits = results[-1]
    D = torch.full(shape, float("nan"), device="cuda")
    torch.cuda.synchronize()
    assert _noalloc(L, D, A, B, C, c, w, splits, null_stream=True) == 0, L.bmm_last_error().decode()
    torch.cuda.synchronize()
    assert np.array_equal(D.cpu().numpy().view(np.uint32), got_prev.view(np.uint32))
    for w, inp, got, splits in results:
        Ao, Bo = oracle.pack(inp["a"], 16), oracle.pack(inp["b"], 8)
        rng = np.random.default_rng(5)
        from tests import util
        idx = util.sample_indices(rng, w.batch, w.M, w.N, 1024)
        ref = oracle.mma_splitk_sampled(Ao, Bo, inp["c_tensor"], inp["c_scalar"], w.dtype,
                                        splits, idx)
        bnd = oracle.bound(Ao, Bo, inp["c_tensor"], inp["c_scalar"], w.dtype, idx)
        Dl = util.tile_to_logical(got)[idx[:, 0], idx[:, 1], idx[:, 2]].astype(np.float64)
        assert (np.abs(Dl - ref) <= gu.BOUND_SCALE * bnd).all(), w.name


def test_noalloc_refuses_more_than_its_scratch():
    """17 partials of 4 MiB exceed the 64 MiB scratch: BMM_ERANGE, D untouched."""
    L = bmm.lib()
    w, _ = CASES[0]
    A = torch.zeros((1, w.M_rep, w.K_rep, 16, 8), dtype=torch.int32, device="cuda")
    B = torch.zeros((1, w.N_rep, w.K_rep, 8, 8), dtype=torch.int32, device="cuda")
    D = torch.full((1, w.M_rep, w.N_rep, 16, 8), 7.0, device="cuda")
    assert _noalloc(L, D, A, B, None, 0.0, w, 17) == ERANGE
    assert "static scratch" in L.bmm_last_error().decode()
    torch.cuda.synchronize()
    assert bool((D == 7.0).all())
