"""museattn_fwd_noalloc (the forward on the library's own per-GPU workspace)
against museattn_fwd (caller workspace): two calls in a row, the second on
a smaller causal input, each compared with the existing entry point on the
same inputs.  Both run the same deterministic kernels, so outputs, lse and
the saved state's labels and retrieval sets must be identical."""
import numpy as np
import pytest

from clustered_approximate_softmax_amd import muse as M
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, N, D, dtype, C, iters, topk, causal, block
    (1, 8, 8, 8192, 64, "bf16", 64, 10, 4, False, 0),     # the 8k acausal workload's shape
    (1, 2, 1, 1000, 128, "bf16", 16, 3, 2, True, 64),     # smaller, causal GQA
]


def _run(case, noalloc):
    import torch
    B, Hq, Hkv, N, D, dtype, C, iters, topk, causal, block = case
    x = gu.gaussian_inputs(B, Hq, Hkv, N, D, dtype, comps=16, seed=N)
    Qd, Kd, Vd = (gu.to_dev(x[k], dtype) for k in "QKV")
    cfg = M.make_cfg(C, iters, topk, causal, block)
    lay = M.layout(B, Hq, Hkv, N, D, M._dt(Qd), cfg)
    assert lay["ws_bytes"] <= 64 << 20
    # zero-filled: entries no problem writes (causal levels label only their
    # segments' rows) then compare equal between the two runs
    st = M.State(torch.zeros(lay["state_bytes"], dtype=torch.uint8, device="cuda"), lay, B, Hq, Hkv, N, D)
    O = torch.empty_like(Qd)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    if noalloc:
        M.museattn_fwd_noalloc(Qd, Kd, Vd, cfg, st, (O, lse))
    else:
        M.museattn_fwd(Qd, Kd, Vd, cfg, state=st, out=(O, lse))
    torch.cuda.synchronize()
    return O, lse, st


def test_noalloc_forward_matches_workspace_forward_twice():
    import torch
    for case in CASES:
        print("case", case, flush=True)
        Oa, la, sa = _run(case, noalloc=True)
        Ob, lb, sb = _run(case, noalloc=False)
        assert torch.equal(Oa, Ob), case
        assert torch.equal(la, lb), case
        for f in ("q_labels", "k_labels", "R", "k_offs", "q_offs"):
            assert torch.equal(sa.field(f), sb.field(f)), (case, f)
        # and within the parity bar of the reference path (identical, so 0)
        assert gu.max_rel(Oa.float().cpu().numpy(), Ob.float().cpu().numpy()) == 0.0
