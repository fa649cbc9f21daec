"""Helpers shared by the GPU parity tests: device tensors from the seeded
generators, the shared-state hand-off to the oracle, and the comparison
criteria (assignments with distance-tie tolerance, retrieval sets with
score-tie tolerance, outputs by max relative error)."""
import numpy as np

from clustered_approximate_softmax_amd import synth

# output tolerances: max |gpu - ref| / max |ref| per (b, h)
TOL = {"f32": 1e-4, "bf16": 2e-2}
TIE = 1e-5     # relative distance / score ties


def to_dev(x32, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)          # exact: values are already bf16
    return t.cuda()


def gaussian_inputs(B, Hq, Hkv, N, D, dtype, comps=16, seed=0, rope=False):
    r = synth.streams(1000 + seed)
    Q = synth.mixture(r["qc"], r["ql"], r["qn"], B, Hq, N, D, comps)
    K = synth.mixture(r["kc"], r["kl"], r["kn"], B, Hkv, N, D, comps)
    if rope:
        Q, K = synth.rope(Q), synth.rope(K)
    V = r["v"].standard_normal((B, Hkv, N, D))
    dO = r["do"].standard_normal((B, Hq, N, D))
    return {k: synth.to_dtype(v, dtype) for k, v in dict(Q=Q, K=K, V=V, dO=dO).items()}


def check_labels(X, mu_prev, labels, tie=TIE):
    """labels must be the nearest centroid of mu_prev (fp64) except at
    relative distance ties; returns the number of tie-tolerated flips."""
    X = np.asarray(X, np.float64)
    mu_prev = np.asarray(mu_prev, np.float64)
    d = np.empty((X.shape[0], mu_prev.shape[0]))
    for r0 in range(0, X.shape[0], 512):
        d[r0:r0 + 512] = ((X[r0:r0 + 512, None, :] - mu_prev[None]) ** 2).sum(-1)
    want = np.argmin(d, axis=1)
    bad = np.nonzero(labels != want)[0]
    for j in bad:
        da, db = d[j, labels[j]], d[j, want[j]]
        assert abs(da - db) <= tie * max(da, db, 1e-30), (j, labels[j], want[j], da, db)
    return len(bad)


def shared_state(state, plan_rows, B, Hq, Hkv, k1w, cq=None):
    """Per-(b, h) dict problem -> (aq, ak, R) read from the GPU state, in the
    form the oracle's forward(shared=...) takes (cq: query clusters, default
    the state's per-problem cluster count)."""
    ql = state.field("q_labels").cpu().numpy()
    kl = state.field("k_labels").cpu().numpy()
    R = state.field("R").cpu().numpy()
    out = {}
    for b in range(B):
        for h in range(Hq):
            g = (h * Hkv) // Hq
            d = {}
            for p, (lev, t, k0, kn, q0, qn) in enumerate(plan_rows):
                aq = ql[lev, b * Hq + h, q0:q0 + qn].astype(np.int64)
                ak = kl[lev, b * Hkv + g, k0:k0 + kn].astype(np.int64)
                Cq = min(R.shape[2] if cq is None else cq, qn)
                Rp = [np.array(sorted(x for x in R[b * Hq + h, p, I] if x >= 0), np.int64) for I in range(Cq)]
                d[p] = (aq, ak, Rp)
            out[(b, h)] = d
    return out


def check_retrieval(results, shared, k1, tie=TIE):
    """GPU retrieval sets are valid top-k1 sets of the oracle's scores."""
    for bh, probs in results.items():
        for p, r in enumerate(probs):
            Rg = shared[bh][p][2]
            for I in range(len(Rg)):
                if r.m[I] == 0:
                    continue
                sig = r.sigma[I]
                valid = np.nonzero(np.isfinite(sig))[0]
                sel = set(Rg[I].tolist())
                assert len(sel) == min(k1, len(valid)), (bh, p, I, sel)
                assert sel <= set(valid.tolist())
                if not sel or len(sel) == len(valid):
                    continue
                lo = min(sig[c] for c in sel)
                hi = max(sig[c] for c in valid if c not in sel)
                assert hi <= lo + tie * max(abs(lo), abs(hi), 1.0), (bh, p, I, lo, hi)


def check_lse(got, ref, dtype, what=""):
    """lse per (batch, head) within the output tolerance relative to the
    largest |lse| of that head: |lse_gpu - lse_ref| <= TOL * max |lse_ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    bound = TOL[dtype] * max(float(np.max(np.abs(ref))), 1e-30)
    err = float(np.max(np.abs(got - ref)))
    assert err <= bound, (what, err, bound)
    return err


def max_rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-30))
