"""GPU parity of museattn_fwd against the oracle.

Attention is compared on shared state: the oracle recomputes every cluster
statistic, summary and output from the GPU's assignments and retrieval
sets.  The retrieval sets themselves must be valid top-k1 sets of the
oracle's scores (ties within 1e-5 relative), and the clustering is checked
separately in lockstep (test_gpu_cluster.py) and here end-to-end against an
oracle run from the same initial points (labels equal except at ties, when
the runs do not diverge)."""
import numpy as np
import pytest

from clustered_approximate_softmax_amd import muse as M
from oracle import muse_oracle as mo
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def run_case(B, Hq, Hkv, N, D, dtype, C, iters, topk, causal=False, block=0, dipole=True, seed=0,
             comps=16, init=False, rope=False, ck=None):
    """C query clusters and ck key clusters (default C)."""
    import torch
    ck = C if ck is None else ck
    x = gu.gaussian_inputs(B, Hq, Hkv, N, D, dtype, comps=comps, seed=seed, rope=rope)
    cfg = M.make_cfg(C, iters, topk, causal, block, dipole, ck=ck)
    ocfg = mo.MuseConfig(cq=C, ck=ck, iters=iters, topk=topk, block=block, causal=causal, dipole=dipole)
    Qd, Kd, Vd = (gu.to_dev(x[k], dtype) for k in "QKV")
    rows = M.plan(N, cfg)
    iq = ik = None
    inits = None
    if init:
        rng = np.random.default_rng(seed + 77)
        iqa = np.stack([gu.synth.draw_inits(rng, [r[5] for r in rows], C) for _ in range(B * Hq)])
        ika = np.stack([gu.synth.draw_inits(rng, [r[3] for r in rows], ck) for _ in range(B * Hkv)])
        iq, ik = torch.from_numpy(iqa).cuda(), torch.from_numpy(ika).cuda()
        inits = {(b, h): {p: (iqa[b * Hq + h, p], ika[b * Hkv + (h * Hkv) // Hq, p])
                          for p in range(len(rows))} for b in range(B) for h in range(Hq)}
    O, lse, st = M.museattn_fwd(Qd, Kd, Vd, cfg, iq, ik)
    torch.cuda.synchronize()
    O = O.float().cpu().numpy()
    lse = lse.cpu().numpy()
    shared = gu.shared_state(st, rows, B, Hq, Hkv, max(1, min(topk, ck)), cq=C)
    Or, Lr, res = mo.forward(x["Q"], x["K"], x["V"], ocfg, shared=shared)
    for b in range(B):
        for h in range(Hq):
            e = gu.max_rel(O[b, h], Or[b, h])
            assert e <= gu.TOL[dtype], (b, h, e)
            gu.check_lse(lse[b, h], Lr[b, h], dtype, (b, h))
    gu.check_retrieval(res, shared, topk)
    return dict(x=x, O=O, lse=lse, state=st, shared=shared, res=res, cfg=cfg, ocfg=ocfg, rows=rows,
                inits=inits, Or=Or)


def test_c1_shape_f32_seeded_init():
    """Acausal, fp32, 1 head, N=1024, D=64, C=16, 10 iterations, no retrieval."""
    r = run_case(1, 1, 1, 1024, 64, "f32", 16, 10, 0, init=True, comps=16)
    # end-to-end clustering vs the oracle from the same starting points
    x, inits = r["x"], r["inits"]
    q0, k0 = inits[(0, 0)][0]
    lab_k, _ = mo.kmeans(x["K"][0, 0], 16, 10, k0[:16])
    ak = r["shared"][(0, 0)][0][1]
    frac = np.mean(ak != lab_k)
    assert frac < 0.01, frac
    # approximation error against exact attention is reported, not bounded tightly
    o, _ = mo.exact_attention(x["Q"][0, 0], x["K"][0, 0], x["V"][0, 0], 1 / 8)
    rse = np.sum((r["O"][0, 0] - o) ** 2) / np.sum(o ** 2)
    assert rse < 1.0


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_acausal_small_retrieval(dtype):
    run_case(1, 2, 2, 1024, 64, dtype, 32, 5, 4, comps=32)


def test_acausal_d128_gqa_chunked_kmeans():
    # N > 2048 exercises the chunked k-means path inside the forward
    run_case(1, 4, 2, 4096, 128, "bf16", 64, 3, 3, comps=32, seed=3)


def test_acausal_ragged_clusters_and_monopole():
    run_case(2, 1, 1, 1000, 64, "bf16", 40, 4, 2, dipole=False, seed=4)


def test_acausal_retrieve_all_is_exact():
    r = run_case(1, 1, 1, 512, 64, "bf16", 16, 3, 16, seed=5)
    x = r["x"]
    o, _ = mo.exact_attention(x["Q"][0, 0], x["K"][0, 0], x["V"][0, 0], 1 / 8)
    assert gu.max_rel(r["O"][0, 0], o) < 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_causal_small(dtype):
    run_case(1, 2, 1, 2048, 64, dtype, 16, 3, 2, causal=True, block=128, seed=6)


def test_causal_ragged_length_tiny_blocks():
    # N not a multiple of the block; level-0 sets smaller than C (C_eff = n)
    run_case(1, 2, 2, 1000, 64, "bf16", 32, 3, 1, causal=True, block=16, seed=7)


@pytest.mark.parametrize("topk", [3, 12])
def test_causal_many_problems_retrieval(topk):
    # 16 heads x 63 problems: enough attention problems for the per-problem
    # score / top-k kernel (one thread per query cluster); sets checked as
    # valid top-k sets of the oracle's scores
    run_case(1, 16, 4, 2048, 64, "bf16", 16, 2, topk, causal=True, block=32, seed=13 + topk)


def test_causal_retrieve_all_is_exact_causal():
    r = run_case(1, 1, 1, 777, 64, "bf16", 8, 2, 8, causal=True, block=64, seed=8)
    x = r["x"]
    o, _ = mo.exact_attention(x["Q"][0, 0], x["K"][0, 0], x["V"][0, 0], 1 / 8, causal=True)
    assert gu.max_rel(r["O"][0, 0], o) < 2e-2


def test_causal_block_covers_sequence():
    r = run_case(1, 1, 1, 300, 128, "bf16", 8, 2, 0, causal=True, block=512, seed=9)
    x = r["x"]
    o, _ = mo.exact_attention(x["Q"][0, 0], x["K"][0, 0], x["V"][0, 0], 1 / np.sqrt(128), causal=True)
    assert gu.max_rel(r["O"][0, 0], o) < 2e-2


def test_causal_monopole():
    run_case(1, 2, 1, 1000, 64, "bf16", 16, 2, 2, causal=True, block=64, dipole=False, seed=15)


def test_fewer_rows_than_clusters():
    # N < C: C_eff = N clusters of one row each; k1 = 3 of them exact, the rest far
    run_case(1, 2, 1, 5, 64, "bf16", 16, 3, 3, seed=11)


def test_single_row():
    run_case(1, 1, 1, 1, 64, "f32", 4, 2, 1, seed=12)


def test_causal_one_block_and_one_row():
    # one level whose only segment has a full key block and a single query row
    run_case(1, 2, 2, 65, 128, "bf16", 8, 2, 2, causal=True, block=64, seed=13)


def test_topk_above_cluster_count_clamps():
    # k1 > C retrieves every non-empty cluster: exact attention
    r = run_case(1, 1, 1, 300, 64, "bf16", 8, 2, 50, seed=14)
    x = r["x"]
    o, _ = mo.exact_attention(x["Q"][0, 0], x["K"][0, 0], x["V"][0, 0], 1 / 8)
    assert gu.max_rel(r["O"][0, 0], o) < 2e-2


def test_forward_is_deterministic():
    import torch
    x = gu.gaussian_inputs(1, 2, 2, 2048, 64, "bf16", comps=32, seed=10)
    cfg = M.make_cfg(32, 4, 2, True, 256)
    Qd, Kd, Vd = (gu.to_dev(x[k], "bf16") for k in "QKV")
    O1, l1, _ = M.museattn_fwd(Qd, Kd, Vd, cfg)
    O2, l2, _ = M.museattn_fwd(Qd, Kd, Vd, cfg)
    torch.cuda.synchronize()
    assert torch.equal(O1, O2) and torch.equal(l1, l2)


@pytest.mark.parametrize("cq,ck,causal,dtype", [(16, 48, False, "bf16"), (64, 24, False, "f32"),
                                                (24, 80, True, "bf16"), (40, 12, True, "bf16")])
def test_separate_query_and_key_cluster_counts(cq, ck, causal, dtype):
    """Queries and keys clustered with their own counts (seeded starting
    points of each side's length), acausal and causal."""
    run_case(1, 4, 2, 3000 if not causal else 2500, 64, dtype, cq, 3, 3, causal=causal,
             block=256 if causal else 0, seed=40 + cq, comps=24, init=True, ck=ck)


def test_large_clusters():
    # clusters of ~250 rows (acausal) and ~512 rows (causal level of span 4096):
    # many contiguous exact tiles per retrieved cluster
    run_case(1, 2, 1, 4000, 64, "bf16", 16, 3, 2, seed=31, comps=16)
    run_case(1, 2, 1, 8192, 64, "bf16", 8, 2, 2, causal=True, block=1024, seed=32, comps=8)


def test_causal_launch_shapes_by_level():
    """Causal GQA levels whose query clusters average 32, 64, 128 and 256
    rows: one-wave workgroups, four waves of one query group, and four
    waves of two query groups, with ragged last segments."""
    run_case(1, 4, 2, 6000, 64, "bf16", 16, 3, 3, causal=True, block=512, seed=51, comps=16)


def test_one_wave_more_exact_chunks_than_the_table():
    """Query clusters of about 32 rows (one-wave workgroups) retrieving six of
    eight key clusters of about 512 rows: more exact 8-row chunks than the
    per-workgroup chunk table holds (256), so tiles are walked from the
    segment list instead."""
    run_case(1, 2, 1, 4096, 64, "bf16", 128, 3, 6, seed=52, comps=16, ck=8)
