"""Pins for the oracle of the causal scheme with spatial blocks, causally
accumulated summaries and two-level retrieval (gist.science page, Technical
Summary, Core Mechanisms: Causal Accumulation, Retrieval-Augmented
Approximation, Exponential Tilting).

Each check compares with something the mathematics fixes:

* retrieving every (cluster, block) pair leaves nothing to approximate:
  exact causal softmax attention;
* far items are exact when a key cluster's keys coincide (zero spread),
  when every key is its own cluster, or when every query is its own
  cluster (nu = q): exact causal attention for any retrieval, which also
  catches a remainder that double counts or drops a retrieved block;
* an output row never depends on values at later positions (values do not
  enter the clustering);
* translating every key by one vector leaves the output unchanged;
* a hand-worked case: the two selections (cluster by summed tilted mass,
  not by count or maximum; then blocks) and the outputs in closed form.
"""
import math

import numpy as np
import pytest

from oracle import muse_oracle as mo
from oracle import muse_v4_oracle as v4


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def exact_causal(Q, K, V, s):
    N = Q.shape[0]
    o = np.zeros((N, V.shape[1]))
    lse = np.zeros(N)
    for i in range(N):
        lg = s * (K[:i + 1] @ Q[i])
        mx = lg.max()
        w = np.exp(lg - mx)
        o[i] = (w @ V[:i + 1]) / w.sum()
        lse[i] = mx + math.log(w.sum())
    return o, lse


def mixture(rng, N, D, comps, sigma=0.3):
    cent = rng.standard_normal((comps, D))
    return cent[rng.integers(0, comps, N)] + sigma * rng.standard_normal((N, D))


def cfg(cq, ck, k1, block, iters=4, scale=0.0):
    return mo.MuseConfig(cq=cq, ck=ck, iters=iters, topk=k1, block=block, causal=True, dipole=True,
                         scale=scale, exact_tilt=True)


@pytest.mark.parametrize("N,Bblk", [(96, 16), (70, 16), (33, 8)])
def test_retrieving_every_pair_is_exact_causal_attention(N, Bblk):
    rng = np.random.default_rng(N)
    D = 8
    Q, K, V = mixture(rng, N, D, 4), mixture(rng, N, D, 4), rng.standard_normal((N, D))
    c = cfg(4, 5, 5, Bblk)
    o, lse, info = v4.forward_head(Q, K, V, c, topk2=v4.n_blocks(N, Bblk))
    eo, el = exact_causal(Q, K, V, c.s(D))
    assert rel(o, eo) < 1e-12 and rel(lse, el) < 1e-12
    # every non-empty earlier (cluster, block) pair was retrieved
    for (I, b), (R1, R2) in info["sel"].items():
        for c_, blocks in zip(R1, R2):
            have = [be for be in range(b) if np.any(info["ak"][be * Bblk:(be + 1) * Bblk] == c_)]
            assert list(blocks) == have


@pytest.mark.parametrize("k1,k2", [(0, 0), (1, 1), (2, 1), (3, 2), (5, 9)])
def test_zero_spread_key_clusters_are_exact(k1, k2):
    """Keys of one cluster coincide: each far item, whatever part of the
    prefix it covers, equals the exact sum over its keys."""
    rng = np.random.default_rng(7 + k1)
    N, D, Bblk, Ck = 90, 6, 10, 5
    base = rng.standard_normal((Ck, D))
    ak = rng.integers(0, Ck, N)
    K = base[ak]
    Q = mixture(rng, N, D, 3)
    V = rng.standard_normal((N, D))
    c = cfg(3, Ck, k1, Bblk)
    aq, _ = v4.cluster_labels(Q, K, c)
    o, lse, _ = v4.forward_head(Q, K, V, c, topk2=k2, shared=dict(aq=aq, ak=ak))
    eo, el = exact_causal(Q, K, V, c.s(D))
    assert rel(o, eo) < 1e-12 and rel(lse, el) < 1e-12


def test_singleton_key_clusters_are_exact():
    rng = np.random.default_rng(3)
    N, D = 40, 5
    Q, K, V = mixture(rng, N, D, 3), rng.standard_normal((N, D)), rng.standard_normal((N, D))
    c = cfg(3, N, 0, 8)
    o, lse, info = v4.forward_head(Q, K, V, c, topk2=0)
    assert len(set(info["ak"].tolist())) == N
    eo, el = exact_causal(Q, K, V, c.s(D))
    assert rel(o, eo) < 1e-12 and rel(lse, el) < 1e-12


@pytest.mark.parametrize("k1,k2", [(0, 0), (2, 1), (1, 3)])
def test_singleton_query_clusters_are_exact(k1, k2):
    """nu_I = q: the tilt is taken at the query itself, so every far item is
    the exact softmax mass and mean of its keys."""
    rng = np.random.default_rng(11 + k2)
    N, D = 48, 6
    Q, K, V = rng.standard_normal((N, D)), mixture(rng, N, D, 4), rng.standard_normal((N, D))
    c = cfg(N, 6, k1, 8)
    o, lse, info = v4.forward_head(Q, K, V, c, topk2=k2)
    assert len(set(info["aq"].tolist())) == N
    eo, el = exact_causal(Q, K, V, c.s(D))
    assert rel(o, eo) < 1e-12 and rel(lse, el) < 1e-12


def test_later_values_do_not_change_earlier_rows():
    rng = np.random.default_rng(5)
    N, D, Bblk = 80, 8, 16
    Q, K, V = mixture(rng, N, D, 4), mixture(rng, N, D, 4), rng.standard_normal((N, D))
    c = cfg(4, 6, 2, Bblk)
    o, lse, _ = v4.forward_head(Q, K, V, c, topk2=1)
    for i in (0, 15, 16, 37, 63, 64):
        V2 = V.copy()
        V2[i + 1:] = rng.standard_normal((N - i - 1, D)) * 5
        o2, lse2, _ = v4.forward_head(Q, K, V2, c, topk2=1)
        assert np.allclose(o2[:i + 1], o[:i + 1], rtol=0, atol=1e-12), i
        assert np.allclose(lse2, lse, rtol=0, atol=1e-12)      # lse never reads values
    # and the approximation is not exact attention here (far items are used)
    eo, _ = exact_causal(Q, K, V, c.s(D))
    assert rel(o, eo) > 1e-6


def test_key_translation_invariance():
    rng = np.random.default_rng(9)
    N, D, Bblk = 64, 8, 16
    Q, K, V = mixture(rng, N, D, 4), mixture(rng, N, D, 4), rng.standard_normal((N, D))
    c = cfg(4, 6, 2, Bblk)
    o, lse, info = v4.forward_head(Q, K, V, c, topk2=1)
    t = 0.7 * rng.standard_normal(D)
    o2, lse2, info2 = v4.forward_head(Q, K + t, V, c, topk2=1)
    assert np.array_equal(info["ak"], info2["ak"])
    assert rel(o2, o) < 1e-10
    # lse shifts by s q.t (the softmax is invariant, its normaliser is not)
    assert np.allclose(lse2 - lse, c.s(D) * (Q @ t), rtol=0, atol=1e-10)


def test_hand_worked_case():
    """D = 2, s = 1, blocks of 2 rows, one query cluster (nu = (1, 0)), key
    clusters given, k1 = k2 = 1.

    Keys: k0 = (2, 0) c0, k1 = (0, 1) c1 | k2 = (1, 0) c0, k3 = (0, -1) c1 |
    k4 = (.5, .5), k5 = (1, 1).  Queries alternate (1, 1), (1, -1).
    Group block 1: prefix = block 0; cluster scores: c0 ln e^2 = 2,
    c1 ln e^0 = 0, so c0 and its block 0 (row 0) are exact; c1's remainder
    is row 1 alone (lnZ 0, kappa k1, U v1).
    Group block 2: c0 ln(e^2 + e) beats c1 ln 2; c0's blocks score 2 and 1:
    block 0 (row 0) exact, c0's far item is row 2 (lnZ 1, kappa (1, 0),
    U v2); c1's is rows 1 and 3 (lnZ ln 2, kappa (0, 0), U (v1 + v3) / 2)."""
    Q = np.array([[1, 1], [1, -1]] * 3, float)
    K = np.array([[2, 0], [0, 1], [1, 0], [0, -1], [.5, .5], [1, 1]], float)
    V = np.array([[j, j * j] for j in range(6)], float)
    c = cfg(1, 2, 1, 2, scale=1.0)
    shared = dict(aq=np.zeros(6, np.int64), ak=np.array([0, 1, 0, 1, 0, 1]))
    o, lse, info = v4.forward_head(Q, K, V, c, topk2=1, shared=shared)
    assert [int(x) for x in info["sel"][(0, 1)][0]] == [0]
    assert [int(x) for x in info["sel"][(0, 1)][1][0]] == [0]
    assert [int(x) for x in info["sel"][(0, 2)][0]] == [0]
    assert [int(x) for x in info["sel"][(0, 2)][1][0]] == [0]
    e = math.e
    v = V
    want = {
        0: ([e ** 2], [v[0]]),
        1: ([e ** 2, e ** -1], [v[0], v[1]]),
        # row 2: exact row 0 (q.k = 2), local row 2 (1), far c1: 0 + (0,1).(0,1) = 1
        2: ([e ** 2, e, e], [v[0], v[2], v[1]]),
        # row 3: exact row 0 (2), local rows 2, 3 (1, 1), far c1: (0,-1).(0,1) = -1
        3: ([e ** 2, e, e, e ** -1], [v[0], v[2], v[3], v[1]]),
        # row 4: exact row 0 (2), local row 4 (1), far c0: 1 + (0,1).(1,0) = 1,
        # far c1: ln 2 + 0
        4: ([e ** 2, e, e, 2.0], [v[0], v[4], v[2], (v[1] + v[3]) / 2]),
        # row 5: exact row 0 (2), local rows 4, 5 (0, 0), far c0: 1 - 0 = 1, far c1: ln 2
        5: ([e ** 2, 1.0, 1.0, e, 2.0], [v[0], v[4], v[5], v[2], (v[1] + v[3]) / 2]),
    }
    for i, (w, vals) in want.items():
        w = np.array(w)
        np.testing.assert_allclose(o[i], (w @ np.array(vals)) / w.sum(), rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(lse[i], math.log(w.sum()), rtol=1e-13)


def test_block_selection_ranks_by_summed_tilted_mass():
    """Within the retrieved cluster, block A holds two keys of tilted logit 1
    (score ln(2e) = 1.69), block B one key of logit 1.5, block C three keys
    of logit 0 (ln 3 = 1.10): k2 = 1 takes A (a maximum would take B, a
    count C), k2 = 2 takes A and B."""
    D, Bblk = 2, 4
    # nu = (1, 0), s = 1: logit = first coordinate
    filler = [-30.0, 0.0]                 # keys of the other cluster, negligible
    rows = []
    lab = []
    blocks = {0: [[1, 0], [1, 0]], 1: [[1.5, 0]], 2: [[0, 0], [0, 0], [0, 0]]}
    for b in range(3):
        ks = blocks[b]
        rows += ks + [filler] * (Bblk - len(ks))
        lab += [0] * len(ks) + [1] * (Bblk - len(ks))
    rows += [[0, 0]] * Bblk               # block 3: the queries
    lab += [1] * Bblk
    K = np.array(rows, float)
    N = K.shape[0]
    Q = np.tile([1.0, 0.0], (N, 1))
    V = np.arange(N * D, dtype=float).reshape(N, D)
    shared = dict(aq=np.zeros(N, np.int64), ak=np.array(lab))
    for k2, want in ((1, [0]), (2, [0, 1]), (3, [0, 1, 2])):
        _, _, info = v4.forward_head(Q, K, V, cfg(1, 2, 1, Bblk, scale=1.0), topk2=k2, shared=shared)
        R1, R2 = info["sel"][(0, 3)]
        assert [int(x) for x in R1] == [0]
        assert [int(x) for x in R2[0]] == want


def test_cluster_selection_clamps_to_non_empty_prefixes():
    """Early blocks see few clusters: k1 larger than the number of key
    clusters present before the block retrieves just those."""
    N, D, Bblk = 24, 2, 4
    K = np.zeros((N, D))
    ak = np.array([0] * 4 + [1] * 4 + [2] * 16)
    K[:, 0] = ak
    Q = np.ones((N, D))
    V = np.ones((N, D))
    _, _, info = v4.forward_head(Q, K, V, cfg(1, 3, 3, Bblk, scale=1.0), topk2=1,
                                 shared=dict(aq=np.zeros(N, np.int64), ak=ak))
    assert [int(x) for x in info["sel"][(0, 1)][0]] == [0]
    assert [int(x) for x in info["sel"][(0, 2)][0]] == [0, 1]
    assert [int(x) for x in info["sel"][(0, 5)][0]] == [0, 1, 2]
