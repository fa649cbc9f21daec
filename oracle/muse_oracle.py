"""Plain, slow, float64 CPU oracle for Multipole Semantic Attention (MuSe).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import this
module: only the test suite, the smoke check and the CPU-baseline leg of the
benchmark do.  It shares no code with the HIP library.

Sources (cited by page and section; the pages are scraped text about
arXiv 2509.10406, "Multipole Semantic Attention: A Fast Approximation of
Softmax Attention for Pretraining", Mitchell and Kersting):

* [GIST-BSC]  gist.science page, Technical Summary, Core Mechanisms,
  "Bidirectional Semantic Clustering": queries and keys are clustered
  separately, each in its own space.
* [GIST-DEC]  same page, Core Mechanisms, "Decomposition": q = centroid +
  residual, k = centroid + residual; of the four terms of the exponent
  (centroid+residual).(centroid+residual) the residual-residual term is the
  only one dropped.
* [GIST-H2S]  same page, Core Mechanisms, "Hierarchical Two-Stage
  Attention" and "Exponential Tilting": query-cluster centroids attend to
  key clusters and give query-cluster-specific summaries (stage 1); each
  query refines with its residual (stage 2).
* [GIST-RAA]  same page, Core Mechanisms, "Retrieval-Augmented
  Approximation": the top-k1 key clusters by tilted summary score are
  attended exactly; the rest go through the summaries.
* [NEWX-ABS]  newx.sg page, "Abstract" (first version): monopole
  (centroid) approximation plus dipole correction; O(NCD) acausal and
  O(NCD log N) causal; causal attention by a hierarchical block
  decomposition with exact local blocks and approximated long-range blocks.

Readings of points the pages leave open (each one listed in the design
document):

* clustering is Lloyd k-means with squared Euclidean distance on the raw
  vectors, a fixed number of iterations, seeded initial points, ties to the
  lowest cluster index, empty clusters keep their previous centroid;
* the softmax scale s multiplies q.k (default 1/sqrt(D)); clustering uses
  the unscaled vectors;
* the dipole of a key cluster c is M_c = sum_j v_j (k_j - mu_c)^T and it is
  evaluated at the query-cluster centroid nu_I (first-order tilt), so the
  tilted summary is T_Ic = S_c + s M_c nu_I with S_c = sum_j v_j; the
  normaliser of the far field is the exact count n_c (the count dipole is
  identically zero);
* the score used for retrieval is sigma_Ic = s nu_I.mu_c + ln n_c (log of the
  monopole tilted mass), ties to the lower cluster index;
* the causal scheme is the dyadic hierarchy of ``causal_plan``.

Parity pins for every function here live in tests/test_oracle_*.py
(brute-force exact limits, closed forms, a direct first-order Taylor check
with its epsilon^2 error law, invariants, scipy's k-means and central finite
differences for the backward).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np


# ----------------------------------------------------------------------------
# Problem configuration
# ----------------------------------------------------------------------------
@dataclass
class MuseConfig:
    """Hyperparameters: the pages say MuSe needs only these (NEWX-ABS)."""

    cq: int = 16          # query clusters per problem (clamped to the set size)
    ck: int = 16          # key clusters per problem (clamped to the set size)
    iters: int = 10       # Lloyd iterations
    topk: int = 0         # k1 retrieved key clusters per query cluster
    block: int = 0        # causal local block size B
    causal: bool = False
    dipole: bool = True   # False: monopole only (T_Ic = S_c)
    scale: float = 0.0    # <= 0 means 1/sqrt(D)
    exact_tilt: bool = False  # True: far items from the exactly tilted summaries (overrides dipole)

    def s(self, D: int) -> float:
        return self.scale if self.scale > 0 else 1.0 / math.sqrt(D)


# ----------------------------------------------------------------------------
# O1: Lloyd k-means, done literally (GIST-BSC; reading: Lloyd, fixed T)
# ----------------------------------------------------------------------------
def sq_dist(X: np.ndarray, mu: np.ndarray, rows: int = 1024) -> np.ndarray:
    """||x_j - mu_c||^2 for every (j, c), summed term by term (no expansion)."""
    X = np.asarray(X, np.float64)
    mu = np.asarray(mu, np.float64)
    out = np.empty((X.shape[0], mu.shape[0]), np.float64)
    for r0 in range(0, X.shape[0], rows):
        diff = X[r0:r0 + rows, None, :] - mu[None, :, :]
        out[r0:r0 + rows] = np.einsum("ncd,ncd->nc", diff, diff)
    return out


def assign_step(X: np.ndarray, mu: np.ndarray) -> np.ndarray:
    """Nearest centroid; np.argmin returns the first (lowest) index on ties."""
    return np.argmin(sq_dist(X, mu), axis=1)


def update_step(X: np.ndarray, labels: np.ndarray, mu_prev: np.ndarray) -> np.ndarray:
    """Mean of each cluster's members; an empty cluster keeps its centroid."""
    X = np.asarray(X, np.float64)
    mu = np.array(mu_prev, np.float64, copy=True)
    for c in range(mu.shape[0]):
        members = X[labels == c]
        if len(members):
            mu[c] = members.sum(axis=0) / len(members)
    return mu


def kmeans(X, C: int, iters: int, init_idx, history: bool = False):
    """Lloyd's algorithm from the points X[init_idx] as starting centroids.

    Returns (labels of the last assignment, centroids after the last
    update[, list of (labels_t, mu_t) for t = 1..iters]).
    """
    X = np.asarray(X, np.float64)
    init_idx = np.asarray(init_idx, np.int64)[:C]
    assert len(set(init_idx.tolist())) == C, "initial indices must be distinct"
    return kmeans_from(X, X[init_idx], iters, history)


def kmeans_from(X, mu0, iters: int, history: bool = False):
    """Lloyd's algorithm from given starting centroids mu0 [C, D]: the
    warm start of a clustering that continues from an earlier call's
    centroids (empty clusters keep their centroid, as in every step)."""
    X = np.asarray(X, np.float64)
    mu = np.array(mu0, np.float64, copy=True)
    labels = np.zeros(X.shape[0], np.int64)
    hist = []
    for _ in range(iters):
        labels = assign_step(X, mu)
        mu = update_step(X, labels, mu)
        if history:
            hist.append((labels.copy(), mu.copy()))
    if history:
        return labels, mu, hist
    return labels, mu


def default_init(n: int, C: int) -> np.ndarray:
    """Evenly spaced starting points floor(c n / C): the library's default."""
    return np.array([(c * n) // C for c in range(C)], np.int64)


# ----------------------------------------------------------------------------
# O2-O4: cluster statistics, scores, retrieval, tilted summaries
# ----------------------------------------------------------------------------
def key_stats(K, V, labels, C):
    """Monopole (n_c, mu_c, S_c) and dipole M_c = sum_j v_j (k_j - mu_c)^T
    of every key cluster (NEWX-ABS: centroid approximation + dipole)."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    D, Dv = K.shape[1], V.shape[1]
    n = np.zeros(C, np.int64)
    mu = np.zeros((C, D))
    S = np.zeros((C, Dv))
    M = np.zeros((C, Dv, D))
    for c in range(C):
        idx = np.nonzero(labels == c)[0]
        n[c] = len(idx)
        if n[c] == 0:
            continue
        mu[c] = K[idx].sum(axis=0) / n[c]
        S[c] = V[idx].sum(axis=0)
        M[c] = V[idx].T @ (K[idx] - mu[c])      # sum of outer products
    return n, mu, S, M


def query_stats(Q, labels, C):
    """Size m_I and centroid nu_I of every query cluster (GIST-DEC)."""
    Q = np.asarray(Q, np.float64)
    m = np.zeros(C, np.int64)
    nu = np.zeros((C, Q.shape[1]))
    for c in range(C):
        idx = np.nonzero(labels == c)[0]
        m[c] = len(idx)
        if m[c]:
            nu[c] = Q[idx].sum(axis=0) / m[c]
    return m, nu


def cluster_scores(nu, mu, n, s):
    """sigma_Ic = s nu_I.mu_c + ln n_c; -inf for empty key clusters.

    exp(sigma_Ic) is the monopole estimate of sum_{j in c} exp(s nu_I.k_j),
    the tilted mass of cluster c seen from query centroid nu_I (GIST-RAA).
    """
    with np.errstate(divide="ignore"):
        logn = np.where(n > 0, np.log(np.maximum(n, 1).astype(np.float64)), -np.inf)
    return s * (np.asarray(nu) @ np.asarray(mu).T) + logn[None, :]


def select_topk(sig_row, k1):
    """The k1 largest scores among non-empty clusters, ties to the lower
    index; returns a sorted array of cluster ids (GIST-RAA, cluster
    selection).  k1 is clamped to the number of non-empty clusters."""
    valid = [c for c in range(len(sig_row)) if np.isfinite(sig_row[c])]
    order = sorted(valid, key=lambda c: (-sig_row[c], c))
    return np.array(sorted(order[:max(0, k1)]), np.int64)


def tilted_summaries(S, M, nu, s, dipole=True):
    """T_Ic = S_c + s M_c nu_I: the value sum of cluster c seen from query
    cluster I, to first order in the tilt exp(s nu_I.(k_j - mu_c))
    (GIST-H2S exponential tilting; NEWX-ABS dipole correction)."""
    T = np.broadcast_to(S[None, :, :], (nu.shape[0],) + S.shape).copy()
    if dipole:
        T += s * np.einsum("cde,Ie->Icd", M, nu)
    return T


def exact_tilt_stats(K, V, labels, Ck, nu, s):
    """Exponentially tilted statistics of every key cluster c seen from every
    query-cluster centroid nu_I (gist.science page, Technical Summary, Core
    Mechanisms, Exponential Tilting: centroids weighted by the attention of
    the query centroid instead of plain averages).  With the tilt weights
    w_j = exp(s nu_I.k_j) over j in c:
      lnZ_Ic   = log sum_j w_j                     (exact log tilted mass)
      kappa_Ic = sum_j w_j k_j / sum_j w_j         (tilted key centroid)
      U_Ic     = sum_j w_j v_j / sum_j w_j         (tilted value mean)
    lnZ is -inf and kappa, U are zero for an empty cluster."""
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    nu = np.asarray(nu, np.float64)
    Cq = nu.shape[0]
    lnZ = np.full((Cq, Ck), -np.inf)
    kap = np.zeros((Cq, Ck, K.shape[1]))
    U = np.zeros((Cq, Ck, V.shape[1]))
    for c in range(Ck):
        idx = np.nonzero(labels == c)[0]
        if len(idx) == 0:
            continue
        lg = s * (nu @ K[idx].T)                     # [Cq, n_c]
        mx = lg.max(axis=1, keepdims=True)
        w = np.exp(lg - mx)
        z = w.sum(axis=1)
        lnZ[:, c] = mx[:, 0] + np.log(z)
        kap[:, c] = (w @ K[idx]) / z[:, None]
        U[:, c] = (w @ V[idx]) / z[:, None]
    return lnZ, kap, U


# ----------------------------------------------------------------------------
# O5: one acausal problem (two stages: far field + exact retrieval)
# ----------------------------------------------------------------------------
@dataclass
class ProblemResult:
    o: np.ndarray              # [n_q, Dv] normalised partial output
    lse: np.ndarray            # [n_q]
    aq: np.ndarray             # query labels
    ak: np.ndarray             # key labels
    R: list                    # retrieved key clusters per query cluster
    n: np.ndarray = None
    mu: np.ndarray = None
    S: np.ndarray = None
    M: np.ndarray = None
    m: np.ndarray = None
    nu: np.ndarray = None
    T: np.ndarray = None
    sigma: np.ndarray = None
    mu_q: np.ndarray = None    # query k-means centroids (== nu where non-empty)
    extra: dict = field(default_factory=dict)


def solve_problem(Q, K, V, s, Cq, Ck, k1, iters, init_q=None, init_k=None,
                  aq=None, ak=None, R=None, dipole=True, qrows=None, exact_tilt=False):
    """One acausal MuSe problem: queries Q [n_q, D] against keys K, V.

    aq/ak/R, when given, replace the clustering and the retrieval (the
    shared-state comparison with the GPU); otherwise they are computed.
    qrows, when given, limits the per-query outputs to those rows (every
    cluster statistic is still taken over the whole problem); the other
    rows of o and lse stay zero.

    exact_tilt: far items use the exactly tilted statistics of
    ``exact_tilt_stats`` instead of the first-order (dipole) summary: for
    query i of cluster I and far cluster c the item has log-weight
    lnZ_Ic + s (q_i - nu_I).kappa_Ic and value U_Ic.  This is the
    decomposition about the query centroid with the key residuals taken
    about the tilted centroid, dropping only the residual cross term
    (q_i - nu_I).(k_j - kappa_Ic); retrieval ranks clusters by the exact
    tilted mass lnZ_Ic.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    nq, nk = Q.shape[0], K.shape[0]
    Cq, Ck = min(Cq, nq), min(Ck, nk)
    mu_q = None
    if ak is None:
        ik = default_init(nk, Ck) if init_k is None else np.asarray(init_k)[:Ck]
        ak, _ = kmeans(K, Ck, iters, ik)
    if aq is None:
        iq = default_init(nq, Cq) if init_q is None else np.asarray(init_q)[:Cq]
        aq, mu_q = kmeans(Q, Cq, iters, iq)
    ak = np.asarray(ak, np.int64)
    aq = np.asarray(aq, np.int64)
    n, mu, S, M = key_stats(K, V, ak, Ck)
    m, nu = query_stats(Q, aq, Cq)
    if exact_tilt:
        lnZ, kap, U = exact_tilt_stats(K, V, ak, Ck, nu, s)
        sig = lnZ.copy()
    else:
        sig = cluster_scores(nu, mu, n, s)
    if R is None:
        R = [select_topk(sig[I], k1) if m[I] > 0 else np.zeros(0, np.int64)
             for I in range(Cq)]
    want = None if qrows is None else np.zeros(nq, bool)
    if want is not None:
        want[np.asarray(qrows, np.int64)] = True
    need = None if want is None else sorted(set(aq[want].tolist()))
    if exact_tilt:
        T = U
    elif need is None:
        T = tilted_summaries(S, M, nu, s, dipole)
    else:
        T = np.zeros((Cq, Ck, S.shape[1]))
        if need:
            T[need] = tilted_summaries(S, M, nu[need], s, dipole)

    Dv = V.shape[1]
    o = np.zeros((nq, Dv))
    lse = np.zeros(nq)
    for I in range(Cq):
        rows = np.nonzero((aq == I) if want is None else ((aq == I) & want))[0]
        if len(rows) == 0:
            continue
        retrieved = [int(c) for c in R[I]]
        ek = np.nonzero(np.isin(ak, retrieved))[0]
        far = np.array([c for c in range(Ck) if n[c] > 0 and c not in retrieved], np.int64)
        # Items of query i: exact keys (weight 1, value v_j) and far clusters
        # (logit s q_i.mu_c, weight n_c, total value T_Ic).  Per GIST-DEC the
        # centroid term, q_i.mu_c and nu_I.(k_j - mu_c) are kept; the residual
        # cross term (q_i - nu_I).(k_j - mu_c) is dropped.
        ell = s * (Q[rows] @ K[ek].T)                      # [r, |ek|]
        if exact_tilt:
            # far items: log-weight lnZ_Ic + s (q_i - nu_I).kappa_Ic, value U_Ic
            lamw = s * ((Q[rows] - nu[I]) @ kap[I, far].T) + lnZ[I, far][None, :]
            logw = np.concatenate([ell, lamw], axis=1)
            if logw.shape[1] == 0:
                continue
            mx = logw.max(axis=1, keepdims=True)
            we = np.exp(ell - mx)
            wf = np.exp(lamw - mx)
            den = we.sum(axis=1) + wf.sum(axis=1)
            num = we @ V[ek] + wf @ U[I, far]
            o[rows] = num / den[:, None]
            lse[rows] = mx[:, 0] + np.log(den)
            continue
        lam = s * (Q[rows] @ mu[far].T)                    # [r, |far|]
        logw = np.concatenate([ell, lam + np.log(n[far].astype(np.float64))[None, :]], axis=1)
        if logw.shape[1] == 0:
            continue
        mx = logw.max(axis=1, keepdims=True)
        we = np.exp(ell - mx)
        wf = np.exp(lam - mx)
        den = we.sum(axis=1) + wf @ n[far].astype(np.float64)
        num = we @ V[ek] + wf @ T[I, far]
        o[rows] = num / den[:, None]
        lse[rows] = mx[:, 0] + np.log(den)
    res = ProblemResult(o=o, lse=lse, aq=aq, ak=ak, R=R, n=n, mu=mu, S=S, M=M,
                        m=m, nu=nu, T=T, sigma=sig, mu_q=mu_q)
    if exact_tilt:
        res.extra.update(lnZ=lnZ, kappa=kap, U=U)
    return res


# ----------------------------------------------------------------------------
# O6/O7: whole calls.  Layout [B, H, N, D]; query head h uses KV head
# floor(h * Hkv / Hq).
# ----------------------------------------------------------------------------
def causal_plan(N: int, Bblk: int):
    """Dyadic block hierarchy (NEWX-ABS: exact local blocks plus long-range
    blocks on log N levels).  Level l has span m = Bblk 2^l; segment t keys
    are rows [2mt, 2mt + m), its queries rows [2mt + m, min(2mt + 2m, N)).
    Returns a list of dicts (level, t, k0, kn, q0, qn) in level-major order.
    """
    nb = -(-N // Bblk)
    L = 0 if nb <= 1 else int(math.ceil(math.log2(nb)))
    plan = []
    for lev in range(L):
        m = Bblk << lev
        t = 0
        while t * 2 * m + m < N:
            k0 = t * 2 * m
            q0 = k0 + m
            plan.append(dict(level=lev, t=t, k0=k0, kn=m, q0=q0, qn=min(m, N - q0)))
            t += 1
    return plan


def acausal_plan(N: int):
    return [dict(level=0, t=0, k0=0, kn=N, q0=0, qn=N)]


def merge_partials(parts):
    """Log-sum-exp merge of normalised partials [(o, lse), ...]."""
    lses = np.stack([p[1] for p in parts])
    top = np.max(lses, axis=0)
    top = np.where(np.isfinite(top), top, 0.0)
    with np.errstate(invalid="ignore", divide="ignore"):
        w = np.exp(lses - top)
        tot = w.sum(axis=0)
        o = sum(w[k][:, None] * parts[k][0] for k in range(len(parts))) / tot[:, None]
        return o, top + np.log(tot)


def local_causal(Q, K, V, s, Bblk, qrows=None):
    """Exact attention of row i over keys [Bblk floor(i/Bblk), i] (only the
    rows in qrows when given)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    N = Q.shape[0]
    o = np.zeros((N, V.shape[1]))
    lse = np.zeros(N)
    if qrows is not None:
        for i in np.asarray(qrows, np.int64):
            b0 = (i // Bblk) * Bblk
            lg = s * (K[b0:i + 1] @ Q[i])
            mx = lg.max()
            p = np.exp(lg - mx)
            o[i] = (p @ V[b0:i + 1]) / p.sum()
            lse[i] = mx + math.log(p.sum())
        return o, lse
    for b0 in range(0, N, Bblk):
        b1 = min(b0 + Bblk, N)
        logits = s * (Q[b0:b1] @ K[b0:b1].T)
        mask = np.tril(np.ones((b1 - b0, b1 - b0), bool))
        logits = np.where(mask, logits, -np.inf)
        mx = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - mx)
        den = p.sum(axis=1, keepdims=True)
        o[b0:b1] = (p @ V[b0:b1]) / den
        lse[b0:b1] = mx[:, 0] + np.log(den[:, 0])
    return o, lse


def forward_head(Qh, Kh, Vh, cfg: MuseConfig, inits=None, shared=None, qrows=None):
    """MuSe for one query head against its KV head: [N, D] each.

    inits:  optional dict problem_index -> (init_q, init_k)
    shared: optional dict problem_index -> (aq, ak, R) from another run
    qrows:  optional absolute query rows; only their outputs are computed
            and problems holding none of them are skipped (None results)
    Returns (o, lse, list of ProblemResult).
    """
    N, D = Qh.shape
    s = cfg.s(D)
    plan = causal_plan(N, cfg.block) if cfg.causal else acausal_plan(N)
    parts_o = np.zeros((len(plan), N, Vh.shape[1]))
    parts_l = np.full((len(plan), N), -np.inf)
    results = []
    qset = None if qrows is None else np.asarray(sorted(set(int(i) for i in qrows)), np.int64)
    for p, pr in enumerate(plan):
        q0, qn, k0, kn = pr["q0"], pr["qn"], pr["k0"], pr["kn"]
        iq, ik = (inits or {}).get(p, (None, None))
        aq, ak, R = (shared or {}).get(p, (None, None, None))
        sub = None
        if qset is not None:
            sub = qset[(qset >= q0) & (qset < q0 + qn)] - q0
            if len(sub) == 0:
                results.append(None)
                continue
        r = solve_problem(Qh[q0:q0 + qn], Kh[k0:k0 + kn], Vh[k0:k0 + kn], s,
                          cfg.cq, cfg.ck, cfg.topk, cfg.iters, iq, ik, aq, ak, R,
                          cfg.dipole, qrows=sub, exact_tilt=cfg.exact_tilt)
        parts_o[p, q0:q0 + qn] = r.o
        parts_l[p, q0:q0 + qn] = r.lse
        results.append(r)
    if not cfg.causal:
        return parts_o[0], parts_l[0], results
    lo, ll = local_causal(Qh, Kh, Vh, s, cfg.block, qrows=qset)
    o, lse = merge_partials([(lo, ll)] + [(parts_o[p], parts_l[p]) for p in range(len(plan))])
    return o, lse, results


def forward(Q, K, V, cfg: MuseConfig, inits=None, shared=None, heads=None):
    """Q [B, Hq, N, D], K/V [B, Hkv, N, D].  Returns O, lse and per-(b, h)
    problem results.  inits/shared are dicts keyed by (b, h) holding the
    per-problem dicts of ``forward_head``.  heads restricts the (b, h)
    pairs computed (others stay zero)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    B, Hq, N, _ = Q.shape
    Hkv = K.shape[1]
    O = np.zeros((B, Hq, N, V.shape[3]))
    L = np.zeros((B, Hq, N))
    res = {}
    for b in range(B):
        for h in range(Hq):
            if heads is not None and (b, h) not in heads:
                continue
            g = (h * Hkv) // Hq
            o, l, r = forward_head(Q[b, h], K[b, g], V[b, g], cfg,
                                   (inits or {}).get((b, h)), (shared or {}).get((b, h)))
            O[b, h], L[b, h], res[(b, h)] = o, l, r
    return O, L, res


def exact_attention(Q, K, V, s, causal=False):
    """Brute-force softmax attention (the quantity MuSe approximates)."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    logits = s * (Q @ np.swapaxes(K, -1, -2))
    if causal:
        N = Q.shape[-2]
        logits = np.where(np.tril(np.ones((N, K.shape[-2]), bool)), logits, -np.inf)
    mx = logits.max(axis=-1, keepdims=True)
    p = np.exp(logits - mx)
    den = p.sum(axis=-1, keepdims=True)
    return (p @ V) / den, (mx + np.log(den))[..., 0]


# ----------------------------------------------------------------------------
# O9: backward with the assignments, retrieval sets and counts held fixed
# ----------------------------------------------------------------------------
def backward_problem(Q, K, V, s, aq, ak, R, Cq, Ck, lse, Delta, dO, dipole=True):
    """Gradient contributions of one acausal problem.

    Every quantity of ``solve_problem`` is differentiated except the labels,
    the retrieval sets and the counts, which are constants.  lse and Delta
    are the final (merged) per-query values, so the same function serves
    the causal parts.  Returns (dQ, dK, dV) for the problem's rows.
    """
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    nq, nk = Q.shape[0], K.shape[0]
    D, Dv = K.shape[1], V.shape[1]
    n, mu, S, M = key_stats(K, V, ak, Ck)
    m, nu = query_stats(Q, aq, Cq)
    T = tilted_summaries(S, M, nu, s, dipole)
    dQ = np.zeros((nq, D))
    dK = np.zeros((nk, D))
    dV = np.zeros((nk, Dv))
    dT = np.zeros((Cq, Ck, Dv))
    dmu = np.zeros((Ck, D))
    for I in range(Cq):
        rows = np.nonzero(aq == I)[0]
        if len(rows) == 0:
            continue
        retrieved = [int(c) for c in R[I]]
        ek = np.nonzero(np.isin(ak, retrieved))[0]
        far = np.array([c for c in range(Ck) if n[c] > 0 and c not in retrieved], np.int64)
        Qr, dOr = Q[rows], dO[rows]
        # exact items: p_ij = exp(l_ij - lse_i), dl_ij = p_ij (dO_i.v_j - Delta_i)
        p = np.exp(s * (Qr @ K[ek].T) - lse[rows, None])
        dl = p * (dOr @ V[ek].T - Delta[rows, None])
        dQ[rows] += s * (dl @ K[ek])
        dK[ek] += s * (dl.T @ Qr)
        dV[ek] += p.T @ dOr
        # far items: rho_ic = exp(lam_ic - lse_i),
        # dlam_ic = rho_ic (dO_i.T_Ic - n_c Delta_i), dT_Ic = sum_i rho_ic dO_i
        rho = np.exp(s * (Qr @ mu[far].T) - lse[rows, None])
        dlam = rho * (dOr @ T[I, far].T - Delta[rows, None] * n[far][None, :])
        dT[I, far] += rho.T @ dOr
        dQ[rows] += s * (dlam @ mu[far])
        dmu[far] += s * (dlam.T @ Qr)
    # through T_Ic = S_c + s M_c nu_I
    dS = dT.sum(axis=0)
    dM = np.zeros((Ck, Dv, D))
    dnu = np.zeros((Cq, D))
    if dipole:
        dM = s * np.einsum("Icd,Ie->cde", dT, nu)
        dnu = s * np.einsum("cde,Icd->Ie", M, dT)
    # through nu_I = mean of its queries
    for I in range(Cq):
        rows = np.nonzero(aq == I)[0]
        if len(rows):
            dQ[rows] += dnu[I] / len(rows)
    # through S_c, M_c = sum v (k - mu)^T and mu_c = mean of its keys
    for c in range(Ck):
        idx = np.nonzero(ak == c)[0]
        if len(idx) == 0:
            continue
        dV[idx] += dS[c][None, :] + (K[idx] - mu[c]) @ dM[c].T
        dK[idx] += (V[idx] - S[c] / n[c]) @ dM[c] + dmu[c][None, :] / n[c]
    return dQ, dK, dV


def local_backward(Q, K, V, s, Bblk, lse, Delta, dO):
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    N = Q.shape[0]
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b0 in range(0, N, Bblk):
        b1 = min(b0 + Bblk, N)
        logits = s * (Q[b0:b1] @ K[b0:b1].T)
        mask = np.tril(np.ones((b1 - b0, b1 - b0), bool))
        p = np.where(mask, np.exp(logits - lse[b0:b1, None]), 0.0)
        dp = dO[b0:b1] @ V[b0:b1].T
        dl = p * (dp - Delta[b0:b1, None])
        dQ[b0:b1] += s * dl @ K[b0:b1]
        dK[b0:b1] += s * dl.T @ Q[b0:b1]
        dV[b0:b1] += p.T @ dO[b0:b1]
    return dQ, dK, dV


def backward(Q, K, V, dO, cfg: MuseConfig, O, lse, results, heads=None):
    """dQ, dK, dV of ``forward`` with labels, retrieval sets and counts
    fixed to those in ``results`` (as returned by forward).  dK and dV sum
    over the query heads that share a KV head."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    dO = np.asarray(dO, np.float64)
    B, Hq, N, D = Q.shape
    Hkv = K.shape[1]
    s = cfg.s(D)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b in range(B):
        for h in range(Hq):
            if heads is not None and (b, h) not in heads:
                continue
            g = (h * Hkv) // Hq
            Delta = np.einsum("nd,nd->n", dO[b, h], np.asarray(O[b, h], np.float64))
            plan = causal_plan(N, cfg.block) if cfg.causal else acausal_plan(N)
            for p, pr in enumerate(plan):
                r = results[(b, h)][p]
                q0, qn, k0, kn = pr["q0"], pr["qn"], pr["k0"], pr["kn"]
                Cq, Ck = min(cfg.cq, qn), min(cfg.ck, kn)
                a, bb, c = backward_problem(Q[b, h, q0:q0 + qn], K[b, g, k0:k0 + kn],
                                            V[b, g, k0:k0 + kn], s, r.aq, r.ak, r.R, Cq, Ck,
                                            lse[b, h, q0:q0 + qn], Delta[q0:q0 + qn],
                                            dO[b, h, q0:q0 + qn], cfg.dipole)
                dQ[b, h, q0:q0 + qn] += a
                dK[b, g, k0:k0 + kn] += bb
                dV[b, g, k0:k0 + kn] += c
            if cfg.causal:
                a, bb, c = local_backward(Q[b, h], K[b, g], V[b, g], s, cfg.block,
                                          lse[b, h], Delta, dO[b, h])
                dQ[b, h] += a
                dK[b, g] += bb
                dV[b, g] += c
    return dQ, dK, dV


def rows_read_by_query_backward(N, cfg: MuseConfig, shared, rows):
    """The query rows whose O and lse ``backward_query_rows`` reads for the
    given rows: the rows themselves plus every member of their query
    cluster in each problem holding them (nu_I couples a cluster's queries)."""
    plan = causal_plan(N, cfg.block) if cfg.causal else acausal_plan(N)
    need = set(int(i) for i in rows)
    for p, pr in enumerate(plan):
        q0, qn = pr["q0"], pr["qn"]
        aq = np.asarray(shared[p][0])
        for i in rows:
            if q0 <= i < q0 + qn:
                need.update(int(q0 + j) for j in np.nonzero(aq == aq[i - q0])[0])
    return np.array(sorted(need), np.int64)


def backward_query_rows(Qh, Kh, Vh, dOh, cfg: MuseConfig, O, lse, shared, rows):
    """dQ of one query head at ``rows`` only, from the same formulas as
    ``backward_problem`` and ``local_backward`` (assignments, retrieval
    sets and counts fixed as in ``shared``: problem -> (aq, ak, R)).  O and
    lse are read only at ``rows_read_by_query_backward``."""
    Qh = np.asarray(Qh, np.float64)
    Kh = np.asarray(Kh, np.float64)
    Vh = np.asarray(Vh, np.float64)
    dOh = np.asarray(dOh, np.float64)
    O = np.asarray(O, np.float64)
    N, D = Qh.shape
    s = cfg.s(D)
    rows = np.asarray(rows, np.int64)
    out = np.zeros((len(rows), D))
    plan = causal_plan(N, cfg.block) if cfg.causal else acausal_plan(N)
    for p, pr in enumerate(plan):
        q0, qn, k0, kn = pr["q0"], pr["qn"], pr["k0"], pr["kn"]
        here = [(k, int(i) - q0) for k, i in enumerate(rows) if q0 <= i < q0 + qn]
        if not here:
            continue
        aq, ak, R = shared[p]
        aq, ak = np.asarray(aq), np.asarray(ak)
        Cq, Ck = min(cfg.cq, qn), min(cfg.ck, kn)
        K, V, Q = Kh[k0:k0 + kn], Vh[k0:k0 + kn], Qh[q0:q0 + qn]
        n, mu, S, M = key_stats(K, V, ak, Ck)
        m, nu = query_stats(Q, aq, Cq)
        T = tilted_summaries(S, M, nu, s, cfg.dipole)
        for I in sorted(set(int(aq[j]) for _, j in here)):
            members = np.nonzero(aq == I)[0]
            retrieved = [int(c) for c in R[I]]
            ek = np.nonzero(np.isin(ak, retrieved))[0]
            far = np.array([c for c in range(Ck) if n[c] > 0 and c not in retrieved], np.int64)
            g = q0 + members
            L = lse[g]
            Delta = np.sum(dOh[g] * O[g], axis=1)
            # dT_I over the far clusters (all members), then dnu_I
            rho = np.exp(s * (Q[members] @ mu[far].T) - L[:, None])
            dT = rho.T @ dOh[g]
            dnu = s * np.einsum("cde,cd->e", M[far], dT) if cfg.dipole else np.zeros(D)
            for k, j in here:
                if aq[j] != I:
                    continue
                jj = int(np.nonzero(members == j)[0][0])
                pe = np.exp(s * (K[ek] @ Q[j]) - L[jj])
                dl = pe * (V[ek] @ dOh[q0 + j] - Delta[jj])
                dlam = rho[jj] * (T[I, far] @ dOh[q0 + j] - Delta[jj] * n[far])
                out[k] += s * (dl @ K[ek]) + s * (dlam @ mu[far]) + dnu / len(members)
    if cfg.causal:
        for k, i in enumerate(rows):
            b0 = (int(i) // cfg.block) * cfg.block
            pe = np.exp(s * (Kh[b0:i + 1] @ Qh[i]) - lse[i])
            dl = pe * (Vh[b0:i + 1] @ dOh[i] - np.dot(dOh[i], O[i]))
            out[k] += s * (dl @ Kh[b0:i + 1])
    return out


def rows_read_by_key_backward(N, cfg: MuseConfig, rows):
    """The query rows whose O and lse ``backward_key_rows`` reads for the
    given key rows: every query of each problem holding one of them as a
    key (the far-field gradients of a key cluster sum over all queries of
    its problem) and, when causal, the rows of its local block at or after
    it."""
    plan = causal_plan(N, cfg.block) if cfg.causal else acausal_plan(N)
    need = set()
    for pr in plan:
        k0, kn, q0, qn = pr["k0"], pr["kn"], pr["q0"], pr["qn"]
        if any(k0 <= int(j) < k0 + kn for j in rows):
            need.update(range(q0, q0 + qn))
    if cfg.causal:
        for j in rows:
            j = int(j)
            b1 = min((j // cfg.block + 1) * cfg.block, N)
            need.update(range(j, b1))
    return np.array(sorted(need), np.int64)


def backward_key_rows(Qg, Kh, Vh, dOg, cfg: MuseConfig, Og, lseg, shared_g, rows):
    """dK and dV of one KV head at key ``rows`` only, summed over the query
    heads that read it, from the same formulas as ``backward_problem`` and
    ``local_backward`` (O9, with assignments, retrieval sets and counts
    fixed as in ``shared_g``).

    Qg, dOg, Og: [G, N, D] of the G query heads of the group; lseg [G, N];
    shared_g: list over those heads of dicts problem -> (aq, ak, R).  O and
    lse are read only at ``rows_read_by_key_backward``.  For key j of cluster
    c in a problem: dV_j = sum_i p_ij dO_i + dS_c + dM_c (k_j - mu_c) and
    dK_j = s sum_i dl_ij q_i + dM_c^T (v_j - S_c / n_c) + dmu_c / n_c, the
    exact sums over the queries whose cluster retrieved c, the cluster
    gradients dS_c, dM_c, dmu_c over the queries that see c as a far item.
    """
    Kh = np.asarray(Kh, np.float64)
    Vh = np.asarray(Vh, np.float64)
    N, D = Kh.shape
    s = cfg.s(D)
    rows = np.asarray(rows, np.int64)
    dK = np.zeros((len(rows), D))
    dV = np.zeros((len(rows), Vh.shape[1]))
    plan = causal_plan(N, cfg.block) if cfg.causal else acausal_plan(N)
    for hq in range(len(Qg)):
        Qh = np.asarray(Qg[hq], np.float64)
        dOh = np.asarray(dOg[hq], np.float64)
        Oh = np.asarray(Og[hq], np.float64)
        lse = np.asarray(lseg[hq], np.float64)
        for p, pr in enumerate(plan):
            q0, qn, k0, kn = pr["q0"], pr["qn"], pr["k0"], pr["kn"]
            here = [(k, int(j) - k0) for k, j in enumerate(rows) if k0 <= j < k0 + kn]
            if not here:
                continue
            aq, ak, R = shared_g[hq][p]
            aq, ak = np.asarray(aq), np.asarray(ak)
            Cq, Ck = min(cfg.cq, qn), min(cfg.ck, kn)
            K, V, Q = Kh[k0:k0 + kn], Vh[k0:k0 + kn], Qh[q0:q0 + qn]
            dO = dOh[q0:q0 + qn]
            L = lse[q0:q0 + qn]
            Delta = np.sum(dO * Oh[q0:q0 + qn], axis=1)
            n, mu, S, M = key_stats(K, V, ak, Ck)
            m, nu = query_stats(Q, aq, Cq)
            T = tilted_summaries(S, M, nu, s, cfg.dipole)
            for c in sorted(set(int(ak[j]) for _, j in here)):
                # queries that retrieved c (exact) and those that see it far
                ret = np.array([I for I in range(Cq) if m[I] > 0 and c in set(int(x) for x in R[I])],
                               np.int64)
                far = np.array([I for I in range(Cq) if m[I] > 0 and I not in set(ret.tolist())],
                               np.int64)
                qe = np.nonzero(np.isin(aq, ret))[0]
                dT = np.zeros((Cq, V.shape[1]))
                dmu = np.zeros(D)
                for I in far:
                    mem = np.nonzero(aq == I)[0]
                    rho = np.exp(s * (Q[mem] @ mu[c]) - L[mem])
                    dlam = rho * (dO[mem] @ T[I, c] - n[c] * Delta[mem])
                    dT[I] = rho @ dO[mem]
                    dmu += s * (dlam @ Q[mem])
                dS = dT.sum(axis=0)
                dM = s * (dT.T @ nu) if cfg.dipole else np.zeros((V.shape[1], D))
                for k, j in here:
                    if ak[j] != c:
                        continue
                    pe = np.exp(s * (Q[qe] @ K[j]) - L[qe])
                    dl = pe * (dO[qe] @ V[j] - Delta[qe])
                    dV[k] += pe @ dO[qe] + dS + dM @ (K[j] - mu[c])
                    dK[k] += s * (dl @ Q[qe]) + dM.T @ (V[j] - S[c] / n[c]) + dmu / n[c]
        if cfg.causal:
            for k, j in enumerate(rows):
                j = int(j)
                b1 = min((j // cfg.block + 1) * cfg.block, N)
                qi = np.arange(j, b1)
                pe = np.exp(s * (Qh[qi] @ Kh[j]) - lse[qi])
                dl = pe * (dOh[qi] @ Vh[j] - np.sum(dOh[qi] * Oh[qi], axis=1))
                dV[k] += pe @ dOh[qi]
                dK[k] += s * (dl @ Qh[qi])
    return dK, dV
