"""moe_permute_noalloc, the entry point for callers that cannot allocate:
bitwise the results of moe_permute, through the C-ABI, on two calls in a
row (the second with a smaller input, so the fixed scratch holds the first
call's values), and its refusal of a cfg whose scratch would not fit."""
import ctypes

import numpy as np
import pytest

import workloads as W
from gpu_parity_helpers import to_dev, to_int

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import expert_router_gemm_softmax_amd as M
    return M


def _permute_both(M, w, seed, slot=False):
    import torch
    cap = None if w.cf is None else M.moe_capacity(w.T, w.k, w.E, w.cf)
    cfg = M.make_cfg(w.T, w.d, w.E, w.k, w.f, w.dtype, capacity=cap,
                     priority="slot" if slot else "token")
    inp = W.make_inputs(w, seed=seed)
    x = to_dev(inp["x"])
    # routing from the library's router on these inputs
    T, E, k, d = w.T, w.E, w.k, w.d
    Rmax = M.moe_rows_max(cfg)
    ws = torch.zeros(M.moe_workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    probs = torch.empty(T, E, dtype=torch.float32, device="cuda")
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    gate = torch.empty(T, k, dtype=torch.float32, device="cuda")
    M.moe_route(cfg, x, to_dev(inp["Wr"]), to_dev(inp["b"]), probs, idx, gate, ws)
    out = []
    for noalloc in (False, True):
        counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
        offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
        row_of = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
        src_of = torch.full((Rmax,), -7, dtype=torch.int32, device="cuda")
        xp = torch.zeros(Rmax, d, dtype=x.dtype, device="cuda")
        if noalloc:
            M.moe_permute_noalloc(cfg, x, idx, counts, offsets, row_of, src_of, xp)
        else:
            M.moe_permute(cfg, x, idx, counts, offsets, row_of, src_of, xp, ws)
        out.append((counts, offsets, row_of, src_of, xp))
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("slot", [False, True], ids=["token-major", "slot-major"])
def test_noalloc_permute_equals_permute_on_two_calls(M, slot):
    import torch
    # c4_large's shape first, then a smaller layer: the second call reads
    # scratch the first one filled with other values
    # (c4_large's routing: its x, Wr and b do not depend on f, kept small here)
    for w, seed in ((W.custom(32768, 4096, 128, 8, 16, dtype="bf16", cf=1.0, bias="normal"), 0),
                    (W.custom(1000, 128, 16, 2, 64, dtype="bf16", cf=1.0, bias="normal"), 3)):
        (c0, o0, r0, s0, x0), (c1, o1, r1, s1, x1) = _permute_both(M, w, seed, slot)
        R = int(to_int(o0)[-1])
        for name, a, b in (("counts", c0, c1), ("offsets", o0, o1), ("row_of", r0, r1)):
            assert torch.equal(a, b), (w.name, name)
        assert torch.equal(s0[:R], s1[:R]) and torch.equal(x0[:R], x1[:R]), w.name
        assert R > 0 and int(to_int(c0).sum()) == w.T * w.k


def test_noalloc_refuses_a_cfg_whose_scratch_does_not_fit(M):
    from expert_router_gemm_softmax_amd import binding as B
    # ceil(T/256) * E * 4 bytes > 4 MiB: nothing is enqueued, clear error
    cfg = M.make_cfg(2 ** 22, 64, 256, 2, 64, "bf16", capacity=None)
    A = 1 << 20
    rc = B.lib.moe_permute_noalloc(ctypes.byref(cfg), A, A, A, A, A, A, A, None)
    assert rc == B.MOE_ERR_WORKSPACE
    assert b"scratch" in B.lib.moe_last_error()
