"""Pins for the oracle's acausal forward (cluster statistics, scores,
retrieval, tilted summaries, two-stage attention).

Each check compares the oracle with something fixed by the mathematics or
by the pages rather than with itself: brute-force softmax in the limits
where MuSe is exact, a directly summed first-order tilt and its epsilon^2
error law, the exactly tilted mean to first order in the scale, invariants
(key translation, linearity in V, constant V), and hand-derived cases.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import muse_oracle as mo

HERE = os.path.dirname(os.path.abspath(__file__))


def exact(Q, K, V, s):
    return mo.exact_attention(Q, K, V, s)


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# -- golden, hand-derived ------------------------------------------------------
def _golden():
    with open(os.path.join(HERE, "golden", "hand_dipole_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_hand_derived_cases(case):
    env = {"exp": math.exp, "log": math.log, "__builtins__": {}}
    Q, K, V = (np.array(case[k], float) for k in ("Q", "K", "V"))
    r = mo.solve_problem(Q, K, V, case["scale"], case["cq"], case["ck"], case["topk"],
                         case["iters"], case["init_q"], case["init_k"])
    assert r.ak.tolist() == case["labels_k"]
    assert [sorted(x.tolist()) for x in r.R] == case["retrieved"]
    want_o = np.array([[eval(e, env) for e in row] for row in case["o"]])
    want_l = np.array([eval(e, env) for e in case["lse"]])
    np.testing.assert_allclose(r.o, want_o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(r.lse, want_l, rtol=1e-13, atol=1e-13)


def _golden_retrieval():
    with open(os.path.join(HERE, "golden", "hand_retrieval_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_retrieval(), ids=lambda c: c["name"])
def test_hand_derived_retrieval_cases(case):
    """The cluster score's log-count and scale each decide a retrieval."""
    env = {"exp": math.exp, "log": math.log, "__builtins__": {}}
    Q, K, V = (np.array(case[k], float) for k in ("Q", "K", "V"))
    r = mo.solve_problem(Q, K, V, case["scale"], case["cq"], case["ck"], case["topk"],
                         case["iters"], case["init_q"], case["init_k"])
    assert r.ak.tolist() == case["labels_k"]
    want_sig = np.array([[eval(e, env) for e in row] for row in case["sigma"]])
    np.testing.assert_allclose(r.sigma, want_sig, rtol=1e-14, atol=1e-14)
    assert [sorted(x.tolist()) for x in r.R] == case["retrieved"]
    want_o = np.array([[eval(e, env) for e in row] for row in case["o"]])
    want_l = np.array([eval(e, env) for e in case["lse"]])
    np.testing.assert_allclose(r.o, want_o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(r.lse, want_l, rtol=1e-13, atol=1e-13)


# -- the retrieval score is the log of the monopole tilted mass -------------------
@pytest.mark.parametrize("seed", range(3))
def test_cluster_score_is_log_tilted_mass_at_zero_spread(seed):
    """With every key of a cluster at its centroid, sigma_Ic is exactly the
    brute-force log sum_{j in c} exp(s nu_I.k_j); with spread, Jensen's
    inequality makes sigma_Ic a lower bound of it."""
    rng = np.random.default_rng(100 + seed)
    D, Ck, Cq = 5, 6, 4
    s = [0.3, 1.0, 2.5][seed]
    centres = rng.standard_normal((Ck, D))
    sizes = rng.integers(1, 9, Ck)
    lab = np.repeat(np.arange(Ck), sizes)
    nu = rng.standard_normal((Cq, D))
    for spread in (0.0, 0.4):
        K = centres[lab] + spread * rng.standard_normal((len(lab), D))
        n, mu, _, _ = mo.key_stats(K, np.zeros_like(K), lab, Ck)
        sig = mo.cluster_scores(nu, mu, n, s)
        for I in range(Cq):
            for c in range(Ck):
                lg = s * (K[lab == c] @ nu[I])
                brute = lg.max() + math.log(np.exp(lg - lg.max()).sum())
                if spread == 0.0:
                    assert abs(sig[I, c] - brute) <= 1e-12 * max(1.0, abs(brute))
                else:
                    assert sig[I, c] <= brute + 1e-12


def test_cluster_score_empty_cluster_is_never_selected():
    n = np.array([3, 0, 2])
    mu = np.array([[0.0, 0.0], [50.0, 0.0], [1.0, 0.0]])
    sig = mo.cluster_scores(np.array([[1.0, 0.0]]), mu, n, 1.0)
    assert sig[0, 1] == -np.inf
    assert mo.select_topk(sig[0], 2).tolist() == [0, 2]
    assert mo.select_topk(sig[0], 5).tolist() == [0, 2]


# -- (a) singleton key clusters reproduce brute-force softmax ---------------------
@pytest.mark.parametrize("seed", range(4))
def test_singleton_key_clusters_are_exact(seed):
    rng = np.random.default_rng(seed)
    nq, nk, D = 40, 24, 8
    Q, K, V = rng.standard_normal((nq, D)), rng.standard_normal((nk, D)), rng.standard_normal((nk, D))
    s = 1 / math.sqrt(D)
    for Cq, k1 in [(1, 0), (5, 0), (7, 3)]:
        r = mo.solve_problem(Q, K, V, s, Cq, nk, k1, 4, init_k=np.arange(nk))
        assert np.all(r.n == 1) and np.allclose(r.M, 0)
        o, lse = exact(Q, K, V, s)
        assert rel(r.o, o) < 1e-13
        np.testing.assert_allclose(r.lse, lse, atol=1e-12)


# -- (b) zero key spread: dipole vanishes, monopole exact -------------------------
def test_zero_key_spread_is_exact():
    rng = np.random.default_rng(11)
    D, C = 6, 5
    centres = rng.standard_normal((C, D)) * 3
    lab = np.repeat(np.arange(C), 9)
    rng.shuffle(lab)
    K = centres[lab]
    V = rng.standard_normal((len(lab), D))
    Q = rng.standard_normal((30, D))
    s = 0.7
    init = np.array([np.nonzero(lab == c)[0][0] for c in range(C)])
    for dip in (True, False):
        r = mo.solve_problem(Q, K, V, s, 4, C, 0, 5, init_k=init, dipole=dip)
        assert np.allclose(r.M, 0, atol=1e-13)
        o, _ = exact(Q, K, V, s)
        assert rel(r.o, o) < 1e-13


# -- (c) dipole = direct first-order Taylor; error law eps^2 vs eps ---------------
def test_tilted_summary_equals_direct_first_order_sum():
    rng = np.random.default_rng(5)
    D, Dv, nk, C = 5, 5, 60, 4
    K, V = rng.standard_normal((nk, D)), rng.standard_normal((nk, Dv))
    ak = rng.integers(0, C, nk)
    nu = rng.standard_normal((3, D))
    s = 0.4
    n, mu, S, M = mo.key_stats(K, V, ak, C)
    T = mo.tilted_summaries(S, M, nu, s)
    for I in range(3):
        for c in range(C):
            want = np.zeros(Dv)
            for j in np.nonzero(ak == c)[0]:
                delta = K[j] - K[ak == c].mean(0)
                want += (1.0 + s * float(np.dot(nu[I], delta))) * V[j]
            np.testing.assert_allclose(T[I, c], want, atol=1e-12)


def _near_field_error(eps, dipole):
    """Queries sit at their cluster centroids, keys at centroid + eps*delta:
    MuSe with k1 = 0 against exact softmax."""
    rng = np.random.default_rng(21)
    D, Cq, Ck, per = 4, 3, 4, 6
    nu = rng.standard_normal((Cq, D))
    mu = rng.standard_normal((Ck, D)) * 2
    delta = rng.standard_normal((Ck * per, D))
    ak = np.repeat(np.arange(Ck), per)
    for c in range(Ck):
        delta[ak == c] -= delta[ak == c].mean(0)
    K = mu[ak] + eps * delta
    aq = np.repeat(np.arange(Cq), 2)
    Q = nu[aq]
    V = rng.standard_normal((len(ak), D))
    s = 0.5
    r = mo.solve_problem(Q, K, V, s, Cq, Ck, 0, 1, aq=aq, ak=ak, dipole=dipole)
    o, _ = exact(Q, K, V, s)
    return np.max(np.abs(r.o - o))


def test_dipole_error_is_second_order():
    e = [_near_field_error(eps, True) for eps in (1e-1, 1e-2, 1e-3)]
    assert 60 < e[0] / e[1] < 160 and 60 < e[1] / e[2] < 160, e
    m = [_near_field_error(eps, False) for eps in (1e-1, 1e-2, 1e-3)]
    assert 6 < m[0] / m[1] < 16 and 6 < m[1] / m[2] < 16, m
    assert e[2] < 1e-2 * m[2]


# -- one key cluster, small scale: first-order tilted mean ------------------------
def test_single_cluster_matches_tilted_mean_to_first_order_in_scale():
    rng = np.random.default_rng(8)
    D, nk = 6, 50
    K, V = rng.standard_normal((nk, D)) + 1.0, rng.standard_normal((nk, D))
    Q = rng.standard_normal((12, D))
    aq = rng.integers(0, 3, 12)
    errs = []
    for s in (1e-2, 1e-3):
        r = mo.solve_problem(Q, K, V, s, 3, 1, 0, 1, aq=aq, ak=np.zeros(nk, int))
        for I in range(3):
            rows = np.nonzero(aq == I)[0]
            if not len(rows):
                continue
            nu = Q[rows].mean(0)
            w = np.exp(s * K @ nu)
            tilted_mean = (w @ V) / w.sum()
            # every query of the cluster gets the same output
            assert np.allclose(r.o[rows], r.o[rows[0]], atol=1e-14)
            errs.append(np.max(np.abs(r.o[rows[0]] - tilted_mean)))
    # error O(s^2): dropping s by 10 drops the error by ~100
    assert max(errs[len(errs) // 2:]) < max(errs[: len(errs) // 2]) / 50


# -- retrieval limits -------------------------------------------------------------
def test_retrieving_every_cluster_is_exact():
    rng = np.random.default_rng(2)
    Q, K, V = rng.standard_normal((50, 8)), rng.standard_normal((70, 8)), rng.standard_normal((70, 8))
    s = 0.35
    r = mo.solve_problem(Q, K, V, s, 6, 9, 9, 5)
    o, lse = exact(Q, K, V, s)
    assert rel(r.o, o) < 1e-13
    np.testing.assert_allclose(r.lse, lse, atol=1e-12)
    r2 = mo.solve_problem(Q, K, V, s, 6, 9, 100, 5)    # k1 clamped
    assert rel(r2.o, o) < 1e-13


def test_topk_selects_largest_scores_with_low_index_ties():
    sig = np.array([0.5, 2.0, -np.inf, 2.0, 1.0, 2.0])
    assert mo.select_topk(sig, 2).tolist() == [1, 3]
    assert mo.select_topk(sig, 4).tolist() == [1, 3, 4, 5]
    assert mo.select_topk(sig, 9).tolist() == [0, 1, 3, 4, 5]
    assert mo.select_topk(sig, 0).tolist() == []


def test_retrieval_improves_on_pure_approximation():
    rng = np.random.default_rng(4)
    Q, K, V = rng.standard_normal((200, 8)), rng.standard_normal((300, 8)), rng.standard_normal((300, 8))
    s = 0.8
    o, _ = exact(Q, K, V, s)
    errs = [np.sum((mo.solve_problem(Q, K, V, s, 8, 16, k1, 6).o - o) ** 2) for k1 in (0, 4, 12, 16)]
    assert errs[0] > errs[1] > errs[2] > errs[3] and errs[3] < 1e-24


# -- invariants --------------------------------------------------------------------
def test_key_translation_invariance():
    rng = np.random.default_rng(9)
    Q, K, V = rng.standard_normal((60, 8)), rng.standard_normal((80, 8)), rng.standard_normal((80, 8))
    t = rng.standard_normal(8) * 3
    a = mo.solve_problem(Q, K, V, 0.4, 5, 7, 2, 6)
    b = mo.solve_problem(Q, K + t, V, 0.4, 5, 7, 2, 6)
    assert np.array_equal(a.ak, b.ak)
    assert rel(b.o, a.o) < 1e-11


def test_linear_in_values_and_constant_values():
    rng = np.random.default_rng(10)
    Q, K = rng.standard_normal((60, 8)), rng.standard_normal((80, 8))
    V1, V2 = rng.standard_normal((80, 8)), rng.standard_normal((80, 8))
    kw = dict(Cq=5, Ck=7, k1=2, iters=6)
    o1 = mo.solve_problem(Q, K, V1, 0.4, **kw).o
    o2 = mo.solve_problem(Q, K, V2, 0.4, **kw).o
    o3 = mo.solve_problem(Q, K, 2.0 * V1 - 3.0 * V2, 0.4, **kw).o
    assert rel(o3, 2.0 * o1 - 3.0 * o2) < 1e-12
    v0 = rng.standard_normal(8)
    oc = mo.solve_problem(Q, K, np.tile(v0, (80, 1)), 0.4, **kw).o
    np.testing.assert_allclose(oc, np.tile(v0, (60, 1)), atol=1e-13)


def test_query_row_permutation_equivariance():
    rng = np.random.default_rng(12)
    Q, K, V = rng.standard_normal((40, 8)), rng.standard_normal((50, 8)), rng.standard_normal((50, 8))
    perm = rng.permutation(40)
    aq = rng.integers(0, 5, 40)
    a = mo.solve_problem(Q, K, V, 0.5, 5, 6, 1, 4, aq=aq)
    b = mo.solve_problem(Q[perm], K, V, 0.5, 5, 6, 1, 4, aq=aq[perm])
    assert rel(b.o, a.o[perm]) < 1e-13


def test_empty_clusters_and_clamps():
    # more clusters than points: clamped; duplicate points leave clusters empty
    Q = np.array([[1.0, 0.0], [1.0, 0.0], [0.0, 1.0]])
    K = np.array([[1.0, 1.0], [1.0, 1.0], [-1.0, 0.0]])
    V = np.array([[1.0, 2.0], [3.0, 4.0], [5.0, 6.0]])
    r = mo.solve_problem(Q, K, V, 1.0, 8, 8, 1, 3)
    assert len(r.n) == 3 and r.n.sum() == 3
    assert np.all(np.isfinite(r.o)) and np.all(np.isfinite(r.lse))
    o, _ = exact(Q, K, V, 1.0)
    # every non-empty key cluster is a point set with zero spread: exact
    assert rel(r.o, o) < 1e-13


def test_forward_gqa_head_mapping():
    rng = np.random.default_rng(13)
    B, Hq, Hkv, N, D = 1, 4, 2, 32, 4
    Q, K, V = (rng.standard_normal((B, h, N, D)) for h in (Hq, Hkv, Hkv))
    cfg = mo.MuseConfig(cq=4, ck=4, iters=3, topk=4)   # all retrieved: exact
    O, L, _ = mo.forward(Q, K, V, cfg)
    for h in range(Hq):
        o, l = exact(Q[0, h], K[0, h // 2], V[0, h // 2], cfg.s(D))
        assert rel(O[0, h], o) < 1e-13
