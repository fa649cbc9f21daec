"""Plain float64 CPU oracle of MuSe's causal scheme with spatial blocks and
causally accumulated summaries (the scheme of the pages' later version).

TEST INFRASTRUCTURE ONLY, like muse_oracle: only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it.  It shares no code
with the HIP library.

Sources (gist.science page, Technical Summary, Core Mechanisms):

* [GIST-CA]  "Causal Accumulation": the sequence is cut into spatial blocks
  and each block sees summaries accumulated over all earlier blocks.
* [GIST-RAA] "Retrieval-Augmented Approximation", two levels: the top-k1
  key clusters by tilted summary score, then inside each of them the top-k2
  spatial blocks; exact attention on the retrieved (cluster, block) pairs
  and on the local block diagonal, summaries for everything else.
* [GIST-H2S] "Exponential Tilting": summaries weighted by the attention of
  the query-cluster centroid (the exactly tilted statistics of
  muse_oracle.exact_tilt_stats, here taken over a key subset).
* [GIST-BSC] queries and keys clustered separately.

Readings (each listed in the design document):

* spatial blocks are the causal local blocks: block b holds rows
  [b B, min((b + 1) B, N)); a query of block b attends exactly to the rows
  of its own block up to itself;
* queries and keys are each clustered once per head over all N rows (the
  acausal clustering); causality enters through the summaries, which only
  ever cover keys of earlier blocks;
* the summaries use the exact exponential tilt at the query-cluster
  centroid nu_I: a key set A gives lnZ = log sum_{j in A} exp(s nu_I.k_j),
  the tilted key mean kappa and the tilted value mean U; a query q of
  cluster I sees A as one item of log-weight lnZ + s (q - nu_I).kappa and
  value U;
* the unit of retrieval is the group (I, b) of the queries of cluster I in
  block b; the cluster score of key cluster c is lnZ over c's keys in blocks
  before b, the block score of (c, beta), beta < b, is lnZ over c's keys in
  block beta; both selections take the largest scores among non-empty sets,
  ties to the lower index, and are clamped to the number of non-empty sets;
* the far item of key cluster c for group (I, b) covers c's keys in blocks
  before b minus the retrieved blocks (the whole prefix when c is not
  retrieved); an empty remainder gives no item;
* queries of block 0 see their local block only.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import muse_oracle as mo


def n_blocks(N: int, Bblk: int) -> int:
    return -(-N // Bblk)


def tilted_set_stats(Kset, Vset, nu, s):
    """(lnZ, kappa, U) of a non-empty key set seen from centroid nu
    (GIST-H2S): w_j = exp(s nu.k_j), lnZ = log sum w, kappa and U the
    w-weighted means of the keys and values."""
    lg = s * (Kset @ nu)
    mx = lg.max()
    w = np.exp(lg - mx)
    z = w.sum()
    return mx + math.log(z), (w @ Kset) / z, (w @ Vset) / z


def set_score(Kset, nu, s):
    """log sum_j exp(s nu.k_j) over a key set; -inf when it is empty."""
    if len(Kset) == 0:
        return -np.inf
    lg = s * (Kset @ nu)
    mx = lg.max()
    return mx + math.log(np.exp(lg - mx).sum())


def cluster_labels(Qh, Kh, cfg: mo.MuseConfig, init_q=None, init_k=None):
    """Per-head clustering over all rows (GIST-BSC): labels of the queries
    (cq clusters) and of the keys (ck clusters), Lloyd from the given or the
    default starting points."""
    N = Qh.shape[0]
    Cq, Ck = min(cfg.cq, N), min(cfg.ck, N)
    iq = mo.default_init(N, Cq) if init_q is None else np.asarray(init_q)[:Cq]
    ik = mo.default_init(N, Ck) if init_k is None else np.asarray(init_k)[:Ck]
    aq, _ = mo.kmeans(Qh, Cq, cfg.iters, iq)
    ak, _ = mo.kmeans(Kh, Ck, cfg.iters, ik)
    return np.asarray(aq, np.int64), np.asarray(ak, np.int64)


def select_group(Kh, ak, nu_I, s, b, Bblk, Ck, k1, k2):
    """Two-level retrieval for the group (I, b) (GIST-RAA): the top-k1 key
    clusters by prefix score, then for each of them the top-k2 earlier
    blocks by block score.  Returns (clusters ascending, list of block
    arrays ascending, one per cluster)."""
    pre = np.arange(b * Bblk)
    sig = np.array([set_score(Kh[pre[ak[pre] == c]], nu_I, s) for c in range(Ck)])
    R1 = mo.select_topk(sig, k1)
    R2 = []
    for c in R1:
        bs = np.array([set_score(Kh[np.arange(be * Bblk, (be + 1) * Bblk)[ak[be * Bblk:(be + 1) * Bblk] == c]],
                                 nu_I, s) for be in range(b)])
        R2.append(mo.select_topk(bs, k2))
    return R1, R2


def forward_head(Qh, Kh, Vh, cfg: mo.MuseConfig, topk2: int, init_q=None, init_k=None, shared=None,
                 qrows=None):
    """Causal MuSe with spatial blocks for one query head against its KV
    head ([N, D] each; cfg.block is the block size, cfg.topk is k1).

    shared: optional dict with labels 'aq', 'ak' used instead of this
            function's own clustering and, optionally, 'R1' =
            {(I, b): (clusters, [blocks per cluster])} used instead of its
            own retrieval (the GPU's state, for parity on shared state).
    qrows:  optional rows; only their outputs are computed.
    Returns (o [N, Dv], lse [N], info) with info holding the labels, the
    query centroids and the retrieval of every group."""
    Qh = np.asarray(Qh, np.float64)
    Kh = np.asarray(Kh, np.float64)
    Vh = np.asarray(Vh, np.float64)
    N, D = Qh.shape
    s = cfg.s(D)
    Bblk = cfg.block
    nb = n_blocks(N, Bblk)
    Cq, Ck = min(cfg.cq, N), min(cfg.ck, N)
    if shared is not None:
        aq = np.asarray(shared["aq"], np.int64)
        ak = np.asarray(shared["ak"], np.int64)
    else:
        aq, ak = cluster_labels(Qh, Kh, cfg, init_q, init_k)
    _, nu = mo.query_stats(Qh, aq, Cq)
    want = np.ones(N, bool) if qrows is None else np.isin(np.arange(N), np.asarray(qrows, np.int64))
    o = np.zeros((N, Vh.shape[1]))
    lse = np.zeros(N)
    sel = {}
    for b in range(nb):
        b0, b1 = b * Bblk, min((b + 1) * Bblk, N)
        for I in range(Cq):
            rows = np.nonzero((aq[b0:b1] == I) & want[b0:b1])[0] + b0
            if len(rows) == 0:
                continue
            if b == 0:
                R1, R2 = np.zeros(0, np.int64), []
            elif shared is not None and "R1" in shared:
                R1, R2 = shared["R1"][(I, b)]
            else:
                R1, R2 = select_group(Kh, ak, nu[I], s, b, Bblk, Ck, cfg.topk, topk2)
            sel[(I, b)] = (R1, R2)
            # exact keys of the retrieved (cluster, block) pairs
            ret = np.zeros(N, bool)
            for c, blocks in zip(R1, R2):
                for be in blocks:
                    r = np.arange(be * Bblk, (be + 1) * Bblk)
                    ret[r[ak[r] == c]] = True
            # far items: per key cluster, its earlier-block keys not retrieved
            far = []
            for c in range(Ck):
                rem = np.nonzero((ak[:b0] == c) & ~ret[:b0])[0]
                if len(rem):
                    far.append(tilted_set_stats(Kh[rem], Vh[rem], nu[I], s))
            ek = np.nonzero(ret)[0]
            for i in rows:
                loc = np.arange(b0, i + 1)
                keys = np.concatenate([ek, loc])
                lg = s * (Kh[keys] @ Qh[i])
                vals = Vh[keys]
                if far:
                    lz = np.array([f[0] for f in far])
                    kap = np.stack([f[1] for f in far])
                    U = np.stack([f[2] for f in far])
                    lg = np.concatenate([lg, lz + s * (kap @ (Qh[i] - nu[I]))])
                    vals = np.concatenate([vals, U])
                mx = lg.max()
                w = np.exp(lg - mx)
                o[i] = (w @ vals) / w.sum()
                lse[i] = mx + math.log(w.sum())
    return o, lse, dict(aq=aq, ak=ak, nu=nu, sel=sel)


def forward(Q, K, V, cfg: mo.MuseConfig, topk2: int, shared=None, heads=None):
    """Q [B, Hq, N, D], K/V [B, Hkv, N, D]; query head h reads KV head
    floor(h Hkv / Hq).  shared: {(b, h): dict for forward_head}."""
    Q = np.asarray(Q, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    B, Hq, N, _ = Q.shape
    Hkv = K.shape[1]
    O = np.zeros((B, Hq, N, V.shape[3]))
    L = np.zeros((B, Hq, N))
    info = {}
    for bb in range(B):
        for h in range(Hq):
            if heads is not None and (bb, h) not in heads:
                continue
            g = (h * Hkv) // Hq
            O[bb, h], L[bb, h], info[(bb, h)] = forward_head(Q[bb, h], K[bb, g], V[bb, g], cfg, topk2,
                                                              shared=(shared or {}).get((bb, h)))
    return O, L, info
