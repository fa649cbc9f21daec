"""Pins for the oracle's causal hierarchy and its fixed-assignment backward.

Causal: the dyadic block decomposition (newx.sg page, Abstract: exact local
blocks, approximated long-range blocks, O(NCD log N)) must cover every pair
j <= i exactly once (brute-force mask count), reduce to exact causal softmax
when every cluster is retrieved or the local block spans the sequence, and
have ceil(log2(ceil(N/B))) levels.

Backward: central finite differences of sum(dO * O) with labels, retrieval
sets and counts frozen, and torch autograd of exact attention in the limit
where MuSe is exact.
"""
import math

import numpy as np
import pytest

from oracle import muse_oracle as mo


@pytest.mark.parametrize("N,B", [(64, 8), (65, 8), (100, 16), (33, 4), (16, 16), (7, 16), (1024, 64)])
def test_causal_plan_covers_each_pair_once(N, B):
    cover = np.zeros((N, N), np.int64)
    for i in range(N):
        b0 = (i // B) * B
        cover[i, b0:i + 1] += 1
    plan = mo.causal_plan(N, B)
    for p in plan:
        cover[p["q0"]:p["q0"] + p["qn"], p["k0"]:p["k0"] + p["kn"]] += 1
        assert p["qn"] > 0 and p["kn"] == B << p["level"]
    assert np.array_equal(cover, np.tril(np.ones((N, N), np.int64)))
    nb = -(-N // B)
    levels = {p["level"] for p in plan}
    assert len(levels) == (0 if nb <= 1 else math.ceil(math.log2(nb)))


def _rand(seed, B=1, Hq=2, Hkv=1, N=40, D=4):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, N, D)), rng.standard_normal((B, Hkv, N, D)),
            rng.standard_normal((B, Hkv, N, D)), rng.standard_normal((B, Hq, N, D)))


def test_causal_all_retrieved_is_exact_causal():
    Q, K, V, _ = _rand(1, N=45)
    cfg = mo.MuseConfig(cq=3, ck=4, iters=3, topk=4, block=4, causal=True)
    O, L, _ = mo.forward(Q, K, V, cfg)
    for h in range(2):
        o, l = mo.exact_attention(Q[0, h], K[0, 0], V[0, 0], cfg.s(4), causal=True)
        np.testing.assert_allclose(O[0, h], o, atol=1e-12)
        np.testing.assert_allclose(L[0, h], l, atol=1e-12)


def test_causal_block_spanning_sequence_is_exact():
    Q, K, V, _ = _rand(2, N=30)
    cfg = mo.MuseConfig(cq=2, ck=2, iters=2, topk=0, block=64, causal=True)
    O, _, res = mo.forward(Q, K, V, cfg)
    assert all(len(r) == 0 for r in res.values())
    o, _ = mo.exact_attention(Q[0, 1], K[0, 0], V[0, 0], cfg.s(4), causal=True)
    np.testing.assert_allclose(O[0, 1], o, atol=1e-12)


def test_causal_approximation_is_close_but_not_exact():
    Q, K, V, _ = _rand(3, N=64, D=8)
    cfg = mo.MuseConfig(cq=4, ck=4, iters=4, topk=1, block=8, causal=True)
    O, _, _ = mo.forward(Q, K, V, cfg)
    o, _ = mo.exact_attention(Q[0, 0], K[0, 0], V[0, 0], cfg.s(8), causal=True)
    # first block is entirely local and exact; later rows are approximate
    np.testing.assert_allclose(O[0, 0, :8], o[:8], atol=1e-12)
    err = np.sum((O[0, 0] - o) ** 2) / np.sum(o ** 2)
    assert 1e-8 < err < 0.5


# -- backward ---------------------------------------------------------------------
def _frozen_forward(Q, K, V, cfg, results):
    shared = {bh: {p: (r.aq, r.ak, r.R) for p, r in enumerate(rs)} for bh, rs in results.items()}
    return mo.forward(Q, K, V, cfg, shared=shared)[0]


def _fd_check(Q, K, V, dO, cfg, h=1e-6, tol=2e-7, samples=12, seed=0):
    O, L, res = mo.forward(Q, K, V, cfg)
    dQ, dK, dV = mo.backward(Q, K, V, dO, cfg, O, L, res)
    rng = np.random.default_rng(seed)
    worst = 0.0
    for name, X, G in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        flat = X.reshape(-1)
        for idx in rng.choice(flat.size, samples, replace=False):
            old = flat[idx]
            flat[idx] = old + h
            fp = np.sum(dO * _frozen_forward(Q, K, V, cfg, res))
            flat[idx] = old - h
            fm = np.sum(dO * _frozen_forward(Q, K, V, cfg, res))
            flat[idx] = old
            fd = (fp - fm) / (2 * h)
            g = G.reshape(-1)[idx]
            worst = max(worst, abs(fd - g) / max(1.0, abs(g)))
            assert abs(fd - g) < tol * max(1.0, abs(g)) + 1e-7, (name, idx, fd, g)
    return worst


@pytest.mark.parametrize("dipole", [True, False])
def test_backward_acausal_matches_finite_differences(dipole):
    Q, K, V, dO = _rand(5, Hq=2, Hkv=1, N=24, D=4)
    cfg = mo.MuseConfig(cq=3, ck=4, iters=3, topk=1, dipole=dipole, scale=0.6)
    _fd_check(Q, K, V, dO, cfg)


def test_backward_causal_gqa_matches_finite_differences():
    Q, K, V, dO = _rand(6, Hq=2, Hkv=1, N=21, D=3)
    cfg = mo.MuseConfig(cq=2, ck=3, iters=2, topk=1, block=4, causal=True, scale=0.7)
    _fd_check(Q, K, V, dO, cfg, samples=10)


def test_backward_exact_limit_equals_softmax_gradient():
    torch = pytest.importorskip("torch")
    Q, K, V, dO = _rand(7, Hq=1, Hkv=1, N=20, D=4)
    cfg = mo.MuseConfig(cq=3, ck=20, iters=2, topk=0, scale=0.5)   # singleton keys
    O, L, res = mo.forward(Q, K, V, cfg)
    dQ, dK, dV = mo.backward(Q, K, V, dO, cfg, O, L, res)
    q, k, v = (torch.tensor(x[0, 0], dtype=torch.float64, requires_grad=True) for x in (Q, K, V))
    out = torch.softmax(0.5 * q @ k.T, dim=-1) @ v
    out.backward(torch.tensor(dO[0, 0]))
    np.testing.assert_allclose(dQ[0, 0], q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dK[0, 0], k.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dV[0, 0], v.grad.numpy(), atol=1e-12)


def test_backward_causal_all_retrieved_equals_causal_softmax_gradient():
    torch = pytest.importorskip("torch")
    Q, K, V, dO = _rand(8, Hq=2, Hkv=1, N=26, D=4)
    cfg = mo.MuseConfig(cq=3, ck=3, iters=2, topk=3, block=4, causal=True, scale=0.5)
    O, L, res = mo.forward(Q, K, V, cfg)
    dQ, dK, dV = mo.backward(Q, K, V, dO, cfg, O, L, res)
    q = torch.tensor(Q[0], dtype=torch.float64, requires_grad=True)
    k = torch.tensor(K[0, 0], dtype=torch.float64, requires_grad=True)
    v = torch.tensor(V[0, 0], dtype=torch.float64, requires_grad=True)
    mask = torch.tril(torch.ones(26, 26, dtype=torch.bool))
    lg = (0.5 * q @ k.T).masked_fill(~mask, float("-inf"))
    out = torch.softmax(lg, dim=-1) @ v
    out.backward(torch.tensor(dO[0]))
    np.testing.assert_allclose(dQ[0], q.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dK[0, 0], k.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dV[0, 0], v.grad.numpy(), atol=1e-12)


def test_row_restricted_forward_equals_full_forward():
    Q, K, V, _ = _rand(9, Hq=1, Hkv=1, N=90, D=4)
    cfg = mo.MuseConfig(cq=3, ck=4, iters=3, topk=1, block=8, causal=True)
    o, l, _ = mo.forward_head(Q[0, 0], K[0, 0], V[0, 0], cfg)
    rows = [0, 7, 8, 33, 64, 89]
    o2, l2, res = mo.forward_head(Q[0, 0], K[0, 0], V[0, 0], cfg, qrows=rows)
    np.testing.assert_allclose(o2[rows], o[rows], atol=1e-13)
    np.testing.assert_allclose(l2[rows], l[rows], atol=1e-13)
    assert any(r is None for r in res)


@pytest.mark.parametrize("causal", [False, True])
def test_row_restricted_query_backward_equals_full_backward(causal):
    Q, K, V, dO = _rand(10, Hq=1, Hkv=1, N=75, D=4)
    cfg = mo.MuseConfig(cq=4, ck=3, iters=3, topk=1, block=8, causal=causal, scale=0.8)
    O, L, res = mo.forward(Q, K, V, cfg)
    dQ, _, _ = mo.backward(Q, K, V, dO, cfg, O, L, res)
    shared = {p: (r.aq, r.ak, r.R) for p, r in enumerate(res[(0, 0)])}
    rows = [0, 9, 16, 40, 74]
    need = mo.rows_read_by_query_backward(75, cfg, shared, rows)
    assert set(rows) <= set(need.tolist())
    # O and lse outside the rows read are poisoned: the result must not change
    Op = np.full_like(O[0, 0], np.nan)
    Lp = np.full_like(L[0, 0], np.nan)
    Op[need], Lp[need] = O[0, 0][need], L[0, 0][need]
    got = mo.backward_query_rows(Q[0, 0], K[0, 0], V[0, 0], dO[0, 0], cfg, Op, Lp, shared, rows)
    np.testing.assert_allclose(got, dQ[0, 0][rows], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_global_identities(causal):
    """Identities of the fixed-assignment MuSe map used as full-size checks:
    probabilities of every row sum to one (sum_j dV_j = sum_i dO_i); a common
    shift of every key leaves each row's logits shifted by a constant
    (sum_j dK_j = 0); O is linear in V (<dV, V> = sum_i dO_i . O_i); and
    O(lam Q, K / lam) = O(Q, K) (<dQ, Q> = <dK, K>), per KV-head group."""
    Q, K, V, dO = _rand(12, B=1, Hq=4, Hkv=2, N=50, D=4)
    cfg = mo.MuseConfig(cq=3, ck=4, iters=2, topk=1, block=8, causal=causal, scale=0.7)
    O, L, res = mo.forward(Q, K, V, cfg)
    dQ, dK, dV = mo.backward(Q, K, V, dO, cfg, O, L, res)
    for g in range(2):
        hs = [h for h in range(4) if (h * 2) // 4 == g]
        np.testing.assert_allclose(dV[0, g].sum(0), sum(dO[0, h].sum(0) for h in hs), atol=1e-10)
        np.testing.assert_allclose(dK[0, g].sum(0), 0.0, atol=1e-10)
        np.testing.assert_allclose(np.sum(dV[0, g] * V[0, g]), sum(np.sum(dO[0, h] * O[0, h]) for h in hs),
                                   rtol=1e-10)
        np.testing.assert_allclose(sum(np.sum(dQ[0, h] * Q[0, h]) for h in hs), np.sum(dK[0, g] * K[0, g]),
                                   rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("causal,dipole", [(False, True), (True, True), (True, False)])
def test_key_row_restricted_backward_equals_full_backward(causal, dipole):
    """dK and dV at chosen key rows, summed over a GQA group, equal the full
    backward's rows, with O and lse poisoned outside the rows it reads."""
    Q, K, V, dO = _rand(13, B=1, Hq=4, Hkv=2, N=83, D=4)
    cfg = mo.MuseConfig(cq=4, ck=3, iters=3, topk=1, block=8, causal=causal, scale=0.8, dipole=dipole)
    O, L, res = mo.forward(Q, K, V, cfg)
    _, dK, dV = mo.backward(Q, K, V, dO, cfg, O, L, res)
    rows = [0, 7, 8, 31, 47, 64, 82]
    need = mo.rows_read_by_key_backward(83, cfg, rows)
    for g in range(2):
        hs = [h for h in range(4) if (h * 2) // 4 == g]
        Op = np.full((len(hs), 83, 4), np.nan)
        Lp = np.full((len(hs), 83), np.nan)
        for k, h in enumerate(hs):
            Op[k, need], Lp[k, need] = O[0, h][need], L[0, h][need]
        shared = [{p: (r.aq, r.ak, r.R) for p, r in enumerate(res[(0, h)])} for h in hs]
        gk, gv = mo.backward_key_rows(Q[0, hs], K[0, g], V[0, g], dO[0, hs], cfg, Op, Lp, shared, rows)
        np.testing.assert_allclose(gk, dK[0, g][rows], atol=1e-12)
        np.testing.assert_allclose(gv, dV[0, g][rows], atol=1e-12)
