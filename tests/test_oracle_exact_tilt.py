"""Pins for the oracle's exact exponential tilt (gist.science page,
Technical Summary, Core Mechanisms: Exponential Tilting, Decomposition).

Each check compares with something the mathematics fixes: a hand-derived
case, exact softmax attention where the expansion is exact (queries at their
cluster centroid, singleton or zero-spread key clusters), agreement with the
first-order (dipole) summary to first order in the scale (the difference
shrinks as s^2), Jensen's inequality between the exact log tilted mass and
the monopole score, and invariance to a common key translation."""
import json
import math
import os

import numpy as np
import pytest

from oracle import muse_oracle as mo

HERE = os.path.dirname(os.path.abspath(__file__))


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def _cases():
    with open(os.path.join(HERE, "golden", "hand_exact_tilt_cases.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_derived_exact_tilt(case):
    env = {"exp": math.exp, "log": math.log, "__builtins__": {}}
    Q, K, V = (np.array(case[k], float) for k in ("Q", "K", "V"))
    r = mo.solve_problem(Q, K, V, case["scale"], case["cq"], case["ck"], case["topk"], case["iters"],
                         case["init_q"], case["init_k"], exact_tilt=True)
    assert r.ak.tolist() == case["labels_k"]
    want_z = np.array([[eval(e, env) for e in row] for row in case["lnZ"]])
    np.testing.assert_allclose(r.extra["lnZ"], want_z, rtol=1e-14, atol=1e-14)
    want_o = np.array([[eval(e, env) for e in row] for row in case["o"]])
    want_l = np.array([eval(e, env) for e in case["lse"]])
    np.testing.assert_allclose(r.o, want_o, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(r.lse, want_l, rtol=1e-13, atol=1e-13)


def _clustered(rng, nq, nk, D, Cq, Ck, spread_q, spread_k):
    cq = rng.standard_normal((Cq, D))
    ck = rng.standard_normal((Ck, D))
    aq = rng.integers(0, Cq, nq)
    ak = np.concatenate([np.arange(Ck), rng.integers(0, Ck, nk - Ck)])
    Q = cq[aq] + spread_q * rng.standard_normal((nq, D))
    K = ck[ak] + spread_k * rng.standard_normal((nk, D))
    V = rng.standard_normal((nk, D))
    return Q, K, V, aq, ak


@pytest.mark.parametrize("seed", range(3))
def test_queries_at_their_centroid_give_exact_attention(seed):
    """q_i = nu_I: each far item is Z_Ic U_Ic = sum_{j in c} exp(s q.k_j) v_j,
    so the output is softmax attention whatever the key spread."""
    rng = np.random.default_rng(300 + seed)
    Q, K, V, aq, ak = _clustered(rng, 40, 60, 6, 5, 7, 0.0, 0.8)
    s = 0.6
    for k1 in (0, 2):
        r = mo.solve_problem(Q, K, V, s, 5, 7, k1, 1, aq=aq, ak=ak, exact_tilt=True)
        o, lse = mo.exact_attention(Q, K, V, s)
        assert rel(r.o, o) < 1e-13
        np.testing.assert_allclose(r.lse, lse, atol=1e-12)


def test_singleton_and_zero_spread_key_clusters_are_exact():
    rng = np.random.default_rng(310)
    Q, K, V, aq, ak = _clustered(rng, 30, 20, 5, 4, 20, 0.7, 0.0)
    s = 0.8
    r = mo.solve_problem(Q, K, V, s, 4, 20, 0, 1, aq=aq, ak=ak, exact_tilt=True)     # singletons
    assert rel(r.o, mo.exact_attention(Q, K, V, s)[0]) < 1e-13
    Q, K, V, aq, ak = _clustered(rng, 30, 50, 5, 4, 6, 0.7, 0.0)                     # zero spread
    r = mo.solve_problem(Q, K, V, s, 4, 6, 0, 1, aq=aq, ak=ak, exact_tilt=True)
    assert rel(r.o, mo.exact_attention(Q, K, V, s)[0]) < 1e-13


def test_agrees_with_the_dipole_to_first_order_in_the_scale():
    """Both expansions share lnZ ~ ln n + s nu.mu, kappa ~ mu and
    U ~ (S + s M nu) / n to first order in s, so their outputs differ by
    O(s^2): shrinking s by 4 shrinks the difference about 16-fold, while
    either one's error against exact attention stays of its own order."""
    rng = np.random.default_rng(320)
    Q, K, V, aq, ak = _clustered(rng, 50, 80, 6, 4, 6, 0.6, 0.6)
    diffs = []
    for s in (0.2, 0.05, 0.0125):
        a = mo.solve_problem(Q, K, V, s, 4, 6, 0, 1, aq=aq, ak=ak, exact_tilt=True)
        b = mo.solve_problem(Q, K, V, s, 4, 6, 0, 1, aq=aq, ak=ak, dipole=True)
        # compare the deviation from the plain value mean, which is O(s)
        vbar = V.mean(axis=0)
        diffs.append(np.max(np.abs(a.o - b.o)) / np.max(np.abs(b.o - vbar)))
    r1, r2 = diffs[0] / diffs[1], diffs[1] / diffs[2]
    assert 3.0 < r1 < 5.5 and 3.0 < r2 < 5.5, diffs    # relative to an O(s) quantity: ratio ~4


def test_exact_log_mass_bounds_the_monopole_score():
    """lnZ_Ic >= s nu_I.mu_c + ln n_c (Jensen), with equality at zero spread."""
    rng = np.random.default_rng(330)
    for spread in (0.0, 0.5):
        Q, K, V, aq, ak = _clustered(rng, 30, 60, 5, 4, 6, 0.5, spread)
        r = mo.solve_problem(Q, K, V, 0.9, 4, 6, 0, 1, aq=aq, ak=ak, exact_tilt=True)
        mono = mo.cluster_scores(r.nu, r.mu, r.n, 0.9)
        if spread == 0.0:
            np.testing.assert_allclose(r.extra["lnZ"], mono, atol=1e-12)
        else:
            assert np.all(r.extra["lnZ"] >= mono - 1e-12)
            assert np.any(r.extra["lnZ"] > mono + 1e-6)


def test_key_translation_invariance():
    rng = np.random.default_rng(340)
    Q, K, V, aq, ak = _clustered(rng, 30, 60, 5, 4, 6, 0.5, 0.5)
    t = rng.standard_normal(5) * 2
    a = mo.solve_problem(Q, K, V, 0.7, 4, 6, 2, 1, aq=aq, ak=ak, exact_tilt=True)
    b = mo.solve_problem(Q, K + t, V, 0.7, 4, 6, 2, 1, aq=aq, ak=ak, exact_tilt=True)
    assert [x.tolist() for x in a.R] == [x.tolist() for x in b.R]
    assert rel(b.o, a.o) < 1e-12


def test_retrieving_every_cluster_is_exact():
    rng = np.random.default_rng(350)
    Q, K, V, aq, ak = _clustered(rng, 30, 60, 5, 4, 6, 0.5, 0.5)
    r = mo.solve_problem(Q, K, V, 0.7, 4, 6, 6, 1, aq=aq, ak=ak, exact_tilt=True)
    assert rel(r.o, mo.exact_attention(Q, K, V, 0.7)[0]) < 1e-13


def test_causal_forward_with_exact_tilt_is_exact_when_all_retrieved():
    rng = np.random.default_rng(360)
    Q, K, V = (rng.standard_normal((1, 1, 70, 4)) for _ in range(3))
    cfg = mo.MuseConfig(cq=3, ck=3, iters=2, topk=3, block=8, causal=True, exact_tilt=True)
    O, _, _ = mo.forward(Q, K, V, cfg)
    o, _ = mo.exact_attention(Q[0, 0], K[0, 0], V[0, 0], 0.5, causal=True)
    assert rel(O[0, 0], o) < 1e-12
