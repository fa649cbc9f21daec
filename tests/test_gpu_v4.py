"""GPU parity of the causal scheme on spatial blocks with causally
accumulated summaries (museattn_fwd with causal = 2) against the oracle of
oracle/muse_v4_oracle.py.

Per (batch, head):
* the block starts v4_qb / v4_kb equal the positions recomputed on the host
  from the GPU's labels (exact integers);
* the retrieval of every group (I, b) is a valid two-level top-k of the
  oracle's fp64 scores: the k1 clusters by ln Z over their keys before block
  b, inside each the k2 blocks by ln Z over that block's keys (ties within
  1e-5 relative), slots past the selection hold -1;
* output and lse equal the oracle's on shared state (the GPU's labels and
  retrieval), to 2e-2 (bf16) or 1e-4 (fp32) of the head's largest value.
Retrieving every (cluster, block) pair is also compared with brute-force
exact causal attention directly."""
import math

import numpy as np
import pytest

from clustered_approximate_softmax_amd import muse as M
from oracle import muse_oracle as mo
from oracle import muse_v4_oracle as v4
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def run(B, Hq, Hkv, N, D, dtype, cq, ck, k1, k2, blk, seed=0, iters=4, comps=16, scale=0.0):
    import torch
    print(f"case B={B} Hq={Hq} Hkv={Hkv} N={N} D={D} {dtype} cq={cq} ck={ck} k1={k1} k2={k2} "
          f"block={blk} seed={seed} scale={scale}", flush=True)
    x = gu.gaussian_inputs(B, Hq, Hkv, N, D, dtype, comps=comps, seed=seed)
    cfg = M.make_cfg(cq, iters, k1, True, blk, ck=ck, blocks=True, topk2=k2, scale=scale)
    Qd, Kd, Vd = (gu.to_dev(x[k], dtype) for k in "QKV")
    O, lse, st = M.museattn_fwd(Qd, Kd, Vd, cfg)
    torch.cuda.synchronize()
    out = dict(x=x, O=O.float().cpu().numpy(), lse=lse.cpu().numpy(), cfg=cfg,
               ql=st.field("q_labels").cpu().numpy()[0], kl=st.field("k_labels").cpu().numpy()[0],
               qperm=st.field("q_perm").cpu().numpy()[0], kperm=st.field("k_perm").cpu().numpy()[0],
               qoffs=st.field("q_offs").cpu().numpy()[:, 0], koffs=st.field("k_offs").cpu().numpy()[:, 0])
    if st.lay["nb"]:
        for n in ("v4_R1", "v4_R2", "v4_kb", "v4_qb"):
            out[n] = st.field(n).cpu().numpy()
    return out


def check_bounds(r, B, Hq, Hkv, N, cq, ck, blk):
    """qb[I][b] = q_offs[I] + #{rows of cluster I before row b blk}, same for keys."""
    nb = -(-N // blk)
    for side, heads, C, lab, offs, name in (("q", B * Hq, cq, r["ql"], r["qoffs"], "v4_qb"),
                                           ("k", B * Hkv, ck, r["kl"], r["koffs"], "v4_kb")):
        for h in range(heads):
            for c in range(min(C, N)):
                rows = np.nonzero(lab[h] == c)[0]
                want = offs[h, c] + np.searchsorted(rows, np.arange(nb + 1) * blk)
                assert np.array_equal(r[name][h, c], want), (side, h, c)


def shared_for(r, b, h, Hq, Hkv, N, blk, cq):
    """The oracle's shared-state dict for head (b, h) from the GPU state."""
    g = (h * Hkv) // Hq
    bh = b * Hq + h
    aq = r["ql"][bh].astype(np.int64)
    ak = r["kl"][b * Hkv + g].astype(np.int64)
    nb = -(-N // blk)
    sel = {}
    for bb in range(1, nb):
        for I in range(min(cq, N)):
            R1 = r["v4_R1"][bh, I, bb]
            R2 = r["v4_R2"][bh, I, bb]
            cl = [int(c) for c in R1 if c >= 0]
            sel[(I, bb)] = (np.array(cl, np.int64),
                            [np.array([int(x) for x in R2[j] if x >= 0], np.int64) for j in range(len(cl))])
    return dict(aq=aq, ak=ak, R1=sel)


def check_selection(r, b, h, Hq, Hkv, N, D, blk, cq, k1, k2, scale, tie=gu.TIE, groups=None):
    """Every group's retrieval (or that of the (I, block) pairs in `groups`)
    is a valid two-level top-k of the fp64 scores."""
    g = (h * Hkv) // Hq
    bh = b * Hq + h
    Qh = r["x"]["Q"][b, h].astype(np.float64)
    Kh = r["x"]["K"][b, g].astype(np.float64)
    aq = r["ql"][bh]
    ak = r["kl"][b * Hkv + g]
    _, nu = mo.query_stats(Qh, aq, min(cq, N))
    nb = -(-N // blk)
    k1w, k2w = r["v4_R1"].shape[3], r["v4_R2"].shape[4]

    def ok_topk(scores, chosen, k, what):
        valid = [i for i in range(len(scores)) if np.isfinite(scores[i])]
        assert len(chosen) == min(k, len(valid)), (what, chosen, valid)
        assert set(chosen) <= set(valid), what
        assert list(chosen) == sorted(chosen), what
        rest = [scores[i] for i in valid if i not in chosen]
        if chosen and rest:
            lo, hi = min(scores[i] for i in chosen), max(rest)
            assert hi <= lo + tie * max(abs(lo), abs(hi), 1.0), (what, lo, hi)

    todo = groups if groups is not None else [(I, bb) for bb in range(1, nb) for I in range(min(cq, N))]
    for I, bb in todo:
        R1 = r["v4_R1"][bh, I, bb]
        if not np.any(aq[bb * blk:(bb + 1) * blk] == I):
            assert np.all(R1 == -1)
            continue
        pre = np.arange(bb * blk)
        sig = [v4.set_score(Kh[pre[ak[pre] == c]], nu[I], scale) for c in range(int(ak.max()) + 1)]
        cl = [int(c) for c in R1 if c >= 0]
        assert np.all(R1[len(cl):] == -1)
        ok_topk(sig, cl, k1, ("clusters", bh, I, bb))
        for j, c in enumerate(cl):
            bs = [v4.set_score(Kh[np.arange(be * blk, (be + 1) * blk)[ak[be * blk:(be + 1) * blk] == c]],
                               nu[I], scale) for be in range(bb)]
            R2 = r["v4_R2"][bh, I, bb, j]
            bl = [int(x) for x in R2 if x >= 0]
            assert np.all(R2[len(bl):] == -1)
            ok_topk(bs, bl, k2, ("blocks", bh, I, bb, c))
        for j in range(len(cl), k1w):
            assert np.all(r["v4_R2"][bh, I, bb, j] == -1)


CASES = [
    # B, Hq, Hkv, N, D, dtype, cq, ck, k1, k2, block
    (1, 2, 1, 1000, 64, "bf16", 8, 16, 2, 2, 64),       # GQA, ragged last block, one-wave groups
    (1, 2, 2, 2048, 128, "f32", 4, 12, 3, 1, 128),      # D = 128 fp32, four-wave groups
    (2, 2, 1, 1536, 64, "bf16", 16, 32, 4, 3, 96),      # batch 2, block not a power of two
    (1, 1, 1, 1024, 64, "f32", 8, 8, 0, 0, 64),         # no retrieval: far items over whole prefixes
    (1, 1, 1, 3000, 64, "bf16", 4, 24, 8, 8, 256),      # wide retrieval, ragged tail
    (1, 2, 1, 777, 128, "bf16", 6, 20, 40, 5, 50),      # k1 clamped to the key clusters
]


@pytest.mark.parametrize("B,Hq,Hkv,N,D,dtype,cq,ck,k1,k2,blk", CASES)
def test_v4_forward_matches_oracle(B, Hq, Hkv, N, D, dtype, cq, ck, k1, k2, blk):
    r = run(B, Hq, Hkv, N, D, dtype, cq, ck, k1, k2, blk, seed=N + cq)
    check_bounds(r, B, Hq, Hkv, N, cq, ck, blk)
    s = 1.0 / math.sqrt(D)
    ocfg = mo.MuseConfig(cq=cq, ck=ck, iters=4, topk=k1, block=blk, causal=True, exact_tilt=True)
    errs = []
    for b in range(B):
        for h in range(Hq):
            check_selection(r, b, h, Hq, Hkv, N, D, blk, cq, k1, k2, s)
            g = (h * Hkv) // Hq
            sh = shared_for(r, b, h, Hq, Hkv, N, blk, cq)
            o, lse, _ = v4.forward_head(r["x"]["Q"][b, h], r["x"]["K"][b, g], r["x"]["V"][b, g], ocfg, k2,
                                        shared=sh)
            e = gu.max_rel(r["O"][b, h], o)
            errs.append(e)
            assert e <= gu.TOL[dtype], (b, h, e)
            gu.check_lse(r["lse"][b, h], lse, dtype, (b, h))
    print("max rel err per head:", [round(e, 6) for e in errs], flush=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_v4_peaked_tilt(dtype):
    """Softmax scale 5: the retrieved blocks often hold nearly all of a
    retrieved cluster's earlier tilted mass, so its far item is taken both
    by subtraction from the prefix (when at least 1/256 remains) and by
    merging the remaining blocks directly (when less does: 17 of the 120
    retrieved (group, cluster) pairs of the fp32 inputs, by the oracle's
    count)."""
    N, D, blk, cq, ck, k1, k2, scale = 1024, 64, 64, 4, 8, 2, 2, 5.0
    r = run(1, 1, 1, N, D, dtype, cq, ck, k1, k2, blk, seed=5, scale=scale)
    check_bounds(r, 1, 1, 1, N, cq, ck, blk)
    check_selection(r, 0, 0, 1, 1, N, D, blk, cq, k1, k2, scale)
    ocfg = mo.MuseConfig(cq=cq, ck=ck, iters=4, topk=k1, block=blk, causal=True, exact_tilt=True, scale=scale)
    sh = shared_for(r, 0, 0, 1, 1, N, blk, cq)
    o, lse, _ = v4.forward_head(r["x"]["Q"][0, 0], r["x"]["K"][0, 0], r["x"]["V"][0, 0], ocfg, k2, shared=sh)
    e = gu.max_rel(r["O"][0, 0], o)
    print("max rel err:", e, flush=True)
    assert e <= gu.TOL[dtype], e
    gu.check_lse(r["lse"][0, 0], lse, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_v4_retrieving_everything_is_exact_attention(dtype):
    """k1 = all key clusters and k2 = all blocks: nothing is approximated."""
    N, D, blk, ck = 1024, 64, 64, 8
    r = run(1, 2, 1, N, D, dtype, 4, ck, ck, N // blk, blk, seed=3)
    s = 1.0 / math.sqrt(D)
    for h in range(2):
        Q = r["x"]["Q"][0, h].astype(np.float64)
        K = r["x"]["K"][0, 0].astype(np.float64)
        V = r["x"]["V"][0, 0].astype(np.float64)
        eo, el = mo.exact_attention(Q[None, None], K[None, None], V[None, None], s, causal=True)[:2]
        e = gu.max_rel(r["O"][0, h], eo[0, 0])
        assert e <= gu.TOL[dtype], (h, e)
        gu.check_lse(r["lse"][0, h], el[0, 0], dtype, h)


def test_v4_single_block_is_local_attention():
    """N <= block: only the local block exists; the output is exact causal
    attention."""
    N, D = 200, 64
    r = run(1, 1, 1, N, D, "f32", 4, 8, 2, 2, 256, seed=4)
    Q, K, V = (r["x"][k][0, 0].astype(np.float64) for k in "QKV")
    eo, el = mo.exact_attention(Q[None, None], K[None, None], V[None, None], 1.0 / math.sqrt(D), causal=True)[:2]
    assert gu.max_rel(r["O"][0, 0], eo[0, 0]) <= gu.TOL["f32"]


def test_v4_is_deterministic():
    import torch
    x = gu.gaussian_inputs(1, 2, 1, 1500, 64, "bf16", seed=9)
    cfg = M.make_cfg(8, 3, 2, True, 100, ck=16, blocks=True, topk2=2)
    Qd, Kd, Vd = (gu.to_dev(x[k], "bf16") for k in "QKV")
    O1, l1, _ = M.museattn_fwd(Qd, Kd, Vd, cfg)
    O2, l2, _ = M.museattn_fwd(Qd, Kd, Vd, cfg)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(l1, l2)
