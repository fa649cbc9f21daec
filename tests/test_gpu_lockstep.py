"""Lockstep check of the clustering inside museattn_fwd.

museattn_fwd clusters the query set and the key set of every problem of a
call (one problem per head when acausal, one per (level, segment) when
causal) in one batch of launches.  The forward is run with t - 1 and with t
Lloyd iterations from the same starting indices; the oracle then takes one
Lloyd step from the GPU's centroids after t - 1 iterations (the starting
points for t = 1).  Labels after t iterations must be the fp64 nearest
centroid except at relative distance ties (1e-5), and the centroids after t
iterations must be the fp64 mean of the GPU's members (an empty cluster
keeps its centroid), so a flip at a tie cannot cascade."""
import numpy as np
import pytest

from clustered_approximate_softmax_amd import muse as M
from oracle import muse_oracle as mo
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _inits(rng, rows, C, heads, side):
    col = 5 if side == "q" else 3      # plan row: (level, t, k0, kn, q0, qn)
    return np.stack([gu.synth.draw_inits(rng, [int(r[col]) for r in rows], C) for _ in range(heads)])


def lockstep_forward(x, B, Hq, Hkv, N, D, dtype, C, iters, topk, causal=False, block=0, heads=None,
                     seed=0, ck=None):
    """Runs the lockstep comparison; returns the number of tie-tolerated
    label flips.  C query clusters, ck key clusters (default C).  heads:
    optional list of (side, head) pairs to check (default: all)."""
    import torch
    ck = C if ck is None else ck
    cnt = {"q": C, "k": ck}
    cfg_rows = M.plan(N, M.make_cfg(C, 1, topk, causal, block, ck=ck))
    rng = np.random.default_rng(seed + 500)
    iq = _inits(rng, cfg_rows, C, B * Hq, "q")
    ik = _inits(rng, cfg_rows, ck, B * Hkv, "k")
    iqd, ikd = torch.from_numpy(iq).cuda(), torch.from_numpy(ik).cuda()
    Qd, Kd, Vd = (gu.to_dev(x[k], dtype) for k in "QKV")
    Xs = {"q": x["Q"].reshape(B * Hq, N, D), "k": x["K"].reshape(B * Hkv, N, D)}
    inits = {"q": iq, "k": ik}
    if heads is None:
        heads = [("q", h) for h in range(B * Hq)] + [("k", g) for g in range(B * Hkv)]
    prev = {}
    for side, h in heads:
        for p, r in enumerate(cfg_rows):
            r0, n = (int(r[4]), int(r[5])) if side == "q" else (int(r[2]), int(r[3]))
            Ce = min(cnt[side], n)
            prev[(side, h, p)] = Xs[side][h, r0:r0 + n][inits[side][h, p, :Ce]].astype(np.float64)
    flips = 0
    for t in range(1, iters + 1):
        cfg = M.make_cfg(C, t, topk, causal, block, ck=ck)
        O, lse, st = M.museattn_fwd(Qd, Kd, Vd, cfg, iqd, ikd)
        torch.cuda.synchronize()
        lab = {"q": st.field("q_labels").cpu().numpy(), "k": st.field("k_labels").cpu().numpy()}
        cent = {"q": st.field("q_cent").cpu().numpy(), "k": st.field("k_cent").cpu().numpy()}
        for side, h in heads:
            for p, r in enumerate(cfg_rows):
                lev = int(r[0])
                r0, n = (int(r[4]), int(r[5])) if side == "q" else (int(r[2]), int(r[3]))
                Ce = min(cnt[side], n)
                X = Xs[side][h, r0:r0 + n]
                a = lab[side][lev, h, r0:r0 + n].astype(np.int64)
                assert a.min() >= 0 and a.max() < Ce, (side, h, p, t)
                flips += gu.check_labels(X, prev[(side, h, p)], a)
                want = mo.update_step(X, a, prev[(side, h, p)])
                got = cent[side][h, p, :Ce].astype(np.float64)
                np.testing.assert_allclose(got, want, rtol=0, atol=3e-6 * max(1.0, np.abs(X).max()),
                                           err_msg=f"{side} head {h} problem {p} iteration {t}")
                prev[(side, h, p)] = got
    return flips


CASES = [
    # B, Hq, Hkv, N, D, dtype, C, iters, topk, causal, block
    (1, 4, 2, 3000, 64, "bf16", 32, 3, 2, False, 0),      # acausal GQA, chunked k-means (n > 2048)
    (2, 1, 1, 1024, 128, "f32", 16, 3, 0, False, 0),      # acausal fp32, batch 2, in-workgroup k-means
    (1, 4, 2, 8192, 64, "bf16", 32, 3, 3, True, 512),     # causal levels 512..4096: both k-means paths
    (1, 4, 1, 2048, 128, "bf16", 16, 3, 2, True, 128),    # causal GQA D=128
    (1, 2, 2, 1000, 64, "bf16", 40, 2, 1, True, 16),      # ragged: level-0 sets smaller than C
]


@pytest.mark.parametrize("B,Hq,Hkv,N,D,dtype,C,iters,topk,causal,block", CASES)
def test_forward_clustering_lockstep(B, Hq, Hkv, N, D, dtype, C, iters, topk, causal, block):
    print(f"case B={B} Hq={Hq} Hkv={Hkv} N={N} D={D} {dtype} C={C} causal={causal} block={block}",
          flush=True)
    x = gu.gaussian_inputs(B, Hq, Hkv, N, D, dtype, comps=max(8, C // 2), seed=N + C)
    flips = lockstep_forward(x, B, Hq, Hkv, N, D, dtype, C, iters, topk, causal, block, seed=N)
    print("tie-tolerated label flips:", flips)


@pytest.mark.parametrize("cq,ck,causal", [(16, 48, False), (40, 12, True)])
def test_forward_clustering_lockstep_separate_counts(cq, ck, causal):
    """Each side clusters with its own count: query labels stay below cq,
    key labels below ck, and both match one oracle Lloyd step."""
    N = 3000
    x = gu.gaussian_inputs(1, 2, 1, N, 64, "bf16", comps=24, seed=cq * ck)
    lockstep_forward(x, 1, 2, 1, N, 64, "bf16", cq, 3, 2, causal, 256 if causal else 0, seed=cq, ck=ck)
