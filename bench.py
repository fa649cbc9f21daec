"""Benchmark of the MuSe hot path on one MI355X.

A step is one museattn_fwd call over the whole workload tensor (all batch x
heads, clustering included; input generation excluded), inputs resident in
HBM; for the training workload (c5) a step is museattn_fwd followed by
museattn_bwd.  Headline workload (default): causal bf16 at the Llama-3.2-1B
attention shape, batch 1, 32 query heads over 8 KV heads, N=65536, D=64,
RoPE, local blocks of 1024, 128 clusters per block level, top-8 retrieval.

Prints one JSON line: ms per layer (median of the timed steps, each
bracketed by HIP events on the launch stream), effective TFLOP/s
(exact-attention FLOPs / time), the roofline of the dominant kernel
(algorithmic work per launch / mean launch time from HIP events around each
launch), exact attention timed on the same GPU (torch SDPA, and this
library's own kernels with every cluster retrieved), the approximation
error (aggregate and mean per-row RSE on sampled rows; the same forward
with the exact exponential tilt in place of the dipole, its time and RSE
beside them), the fp64 oracle
timed on a bounded sample on the host cores, and a sweep over the other
workloads (8k acausal, 16k causal batch 4, 64k D=128 forward + backward)
with the same timing, SDPA, RSE and CPU-baseline figures.
"""
import argparse
import gc
import json
import re
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MuSe attn ms/layer + effective TFLOP/s (% of MFMA peak) at N=8k..64k, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
HEADLINE = "c4"
BLOCKS_K2 = 4      # blocks retrieved inside each retrieved cluster (spatial-block scheme)
SWEEP = ("c2", "c3", "c5")


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default=HEADLINE, choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--no-sweep", action="store_true", help="time the headline workload only")
    ap.add_argument("--sweep-steps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work per workload (bounded sample)")
    ap.add_argument("--no-exact", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--no-blocks", action="store_true", help="skip the spatial-block scheme entry")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="also run a plain copy of this many MiB (for PMC byte-counter scaling)")
    return ap.parse_args()


def exact_flops(w):
    """Exact softmax-attention FLOPs of the step (forward: QK^T and PV;
    backward adds five products of the same size: x 3.5 for fwd + bwd)."""
    f = 4.0 * w.B * w.Hq * w.D * (w.N * (w.N + 1) / 2 if w.causal else w.N * w.N)
    return 3.5 * f if w.backward else f


def kernel_models(w, M, st, rows):
    """Algorithmic work per call for each kernel name: (flops, bytes, bound)."""
    C, D, T = w.C, w.D, w.iters
    eb = 2 if w.dtype == "bf16" else 4
    qoffs = st.field("q_offs").cpu().numpy()
    koffs = st.field("k_offs").cpu().numpy()
    R = st.field("R").cpu().numpy()
    BHq, BHk = w.B * w.Hq, w.B * w.Hkv
    sizes = [(int(r[3]), int(r[5])) for r in rows]     # (kn, qn)
    pts_q = sum(qn for _, qn in sizes) * BHq
    pts_k = sum(kn for kn, _ in sizes) * BHk
    km = {}
    # Lloyd distances: 2 n C D per point per iteration (Q and K sets)
    large_q = sum(qn for kn, qn in sizes if qn > 2048) * BHq
    large_k = sum(kn for kn, qn in sizes if kn > 2048) * BHk
    small = (pts_q - large_q) + (pts_k - large_k)
    large = large_q + large_k
    km["km_local"] = (2.0 * small * C * D * T, small * D * eb * T, "mfma")
    # assignment reads every point once per iteration: intensity C flop/B, below the bf16
    # ridge, so it is priced against HBM
    km["km_assign"] = (2.0 * large * C * D * T, large * D * eb * T, "hbm")
    # retrieved keys and far clusters summed over every query of every problem
    m = np.diff(qoffs, axis=-1).astype(np.float64)                       # [BHq, P, C]
    kvmap = np.array([(bh // w.Hq) * w.Hkv + (bh % w.Hq) * w.Hkv // w.Hq for bh in range(BHq)])
    cnt = np.diff(koffs, axis=-1)[kvmap].astype(np.float64)              # [BHq, P, C]
    Rc = np.clip(R, 0, None)
    rsz = np.take_along_axis(cnt[:, :, None, :].repeat(R.shape[2], 2), Rc, axis=3) * (R >= 0)
    ret = float((m * rsz.sum(-1)).sum())
    nz = (cnt > 0).sum(-1)                                               # [BHq, P]
    nsel = (R >= 0).sum(-1)                                              # [BHq, P, C]
    far = float((m * (nz[:, :, None] - nsel)).sum())
    attn_flops = 2.0 * (ret + far) * (D + D)
    attn_bytes = (pts_q * D * eb * 2) + ret / max(1, pts_q) * 0  # Q in, O out
    name = "attn_level" if w.causal else "attn_far_retrieve"
    km[name] = (attn_flops, attn_bytes, "mfma")
    km["summarize"] = (2.0 * pts_k * D * D, pts_k * 2 * D * eb, "hbm")
    Pn = len(rows)
    km["tilt"] = (2.0 * BHq * Pn * C * C * D * D, BHq * Pn * C * C * D * 4, "hbm")
    if w.causal:
        km["attn_local"] = (2.0 * BHq * w.N * (w.block + 1) / 2 * 2 * D, BHq * w.N * D * eb * 2, "mfma")
    if w.backward:
        # per (query, item) pair: S and dP, then dQ (query-centric) or dK and dV (item-centric)
        loc = BHq * w.N * (w.block + 1) / 2 if w.causal else 0.0
        km["bwd_q"] = (6.0 * D * (ret + far), pts_q * D * eb * 3, "mfma")
        km["bwd_kv"] = (8.0 * D * ret, pts_k * D * eb * 4, "mfma")
        km["bwd_far"] = (8.0 * D * far, BHq * Pn * C * C * D * 4 * 2, "mfma")
        km["bwd_q_local"] = (6.0 * D * loc, BHq * w.N * D * eb * 3, "mfma")
        km["bwd_kv_local"] = (8.0 * D * loc, BHq * w.N * D * eb * 2, "mfma")
        # dM and dnu contractions (C x C x D x D per problem each), reductions and broadcasts
        km["bwd_dM"] = (2.0 * BHq * Pn * C * C * D * D, BHq * Pn * C * C * D * 4, "mfma")
        km["bwd_dnu"] = (2.0 * BHq * Pn * C * C * D * D, BHq * Pn * C * C * D * 4, "mfma")
        km["bwd_reduce_k"] = (0.0, BHq * Pn * C * C * D * 4 * 2, "hbm")
        km["bwd_spread_q"] = (0.0, pts_q * D * 4 * 2, "hbm")
        km["bwd_bcast_k"] = (4.0 * pts_k * D * D, pts_k * D * (eb * 2 + 4 * 4), "mfma")
        f, b_, bd = km["tilt"]
        km["tilt"] = (2 * f, 2 * b_, bd)          # recomputed once in the backward
    return km


def measured_traffic(w, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of this workload (scaled by the copy calibration), or
    None when there is none or the kernel's source changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{'c' + str(w.number)}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get("kernels", {}).get(kernel)
    if not rec:
        return None
    h = hashlib.sha256()
    for f in (rec["source"], "common.h"):
        with open(os.path.join(ROOT, "clustered_approximate_softmax_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != rec["source_sha"]:
        return None
    return int(rec["bytes_per_dispatch"])


def time_steps(fn, steps, torch):
    """Run `steps` calls of fn, each bracketed by HIP events on the current
    (launch) stream, the whole region bracketed by device synchronisation.
    Returns (median ms per call from the events, mean ms per call from the
    host clock around the region)."""
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    t0 = time.perf_counter()
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    per = [a.elapsed_time(b) for a, b in evs]
    return float(np.median(per)), wall


def exact_attention_ms(Q, K, V, w, steps, torch):
    """torch SDPA on the same tensors (KV heads repeated for GQA); for the
    training workload forward + backward, restricted to the fused flash /
    memory-efficient kernels (no math fallback).  Median ms per call."""
    import torch.nn.functional as F
    from torch.nn.attention import SDPBackend, sdpa_kernel
    Hq, Hkv = w.Hq, w.Hkv
    Kx = (K.repeat_interleave(Hq // Hkv, dim=1) if Hq != Hkv else K).contiguous()
    Vx = (V.repeat_interleave(Hq // Hkv, dim=1) if Hq != Hkv else V).contiguous()
    if w.backward:
        q, k, v = (t.detach().clone().requires_grad_(True) for t in (Q, Kx, Vx))
        go = torch.randn_like(q)

        def f():
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
                o = F.scaled_dot_product_attention(q, k, v, is_causal=w.causal)
                o.backward(go)
    else:
        def f():
            F.scaled_dot_product_attention(Q, Kx, Vx, is_causal=w.causal)
    for _ in range(2):
        f()
    return time_steps(f, steps, torch)[0]


def own_exact_ms(Q, K, V, w, M, steps, torch):
    """The same forward with k1 = C: every key cluster is retrieved, so the
    gathered exact kernels compute plain softmax attention (clustering and
    summaries included).  Returns (median ms per call, O)."""
    cfg = M.make_cfg(w.C, w.iters, w.C, w.causal, w.block)
    O, lse, st = M.museattn_fwd(Q, K, V, cfg)
    ws = torch.empty(M.layout(w.B, w.Hq, w.Hkv, w.N, w.D, M._dt(Q), cfg)["ws_bytes"], dtype=torch.uint8,
                     device="cuda")

    def f():
        M.museattn_fwd(Q, K, V, cfg, state=st, ws=ws, out=(O, lse))
    f()
    ms = time_steps(f, steps, torch)[0]
    del ws, st, lse
    return ms, O


def rse_vs_exact(Q, K, V, O, w, torch, rows_per_head=1024):
    """||O - O_exact||^2 / ||O_exact||^2 on sampled query rows (fp32 exact),
    and the mean over those rows of the per-row ratio."""
    g = torch.Generator(device="cpu").manual_seed(0)
    num = den = 0.0
    rows = []
    s = 1.0 / math.sqrt(w.D)
    for b in range(w.B):
        for h in range(w.Hq):
            kv = h * w.Hkv // w.Hq
            idx = torch.randperm(w.N, generator=g)[:rows_per_head].sort().values.cuda()
            q = Q[b, h, idx].float()
            k = K[b, kv].float()
            v = V[b, kv].float()
            lg = (q @ k.T) * s
            if w.causal:
                mask = torch.arange(w.N, device=q.device)[None, :] > idx[:, None]
                lg = lg.masked_fill(mask, float("-inf"))
            ex = torch.softmax(lg, dim=-1) @ v
            err = ((O[b, h, idx].float() - ex) ** 2).sum(-1)
            ref = (ex ** 2).sum(-1)
            num += float(err.sum())
            den += float(ref.sum())
            rows.append((err / ref.clamp_min(1e-30)).cpu())
    return num / den, float(torch.cat(rows).mean())


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(w, x, budget_s):
    """The fp64 oracle timed on a bounded sample of the workload, scaled to
    the whole layer.

    Acausal: whole (batch, query head) problems until the budget is spent,
    extrapolated linearly in the number of heads.  Causal: the first segment
    of each block level of head 0 (forward, plus the backward for a training
    workload), timed level by level while the budget is predicted to last (a
    level costs about twice the one below it); each
    larger level is extrapolated from the largest measured one linearly in
    the span (every step of a problem, k-means, statistics and attention, is
    linear in its row count at fixed C and D); each level's time is
    multiplied by its segment count, the exact local blocks by the block
    count from four timed blocks, and the head by B * Hq."""
    from oracle import muse_oracle as mo
    cfg = mo.MuseConfig(cq=w.C, ck=w.C, iters=w.iters, topk=w.topk, block=w.block, causal=w.causal)
    Q, K, V = x["Q"], x["K"], x["V"]
    dO = x.get("dO")
    s = cfg.s(w.D)
    heads = w.B * w.Hq

    def one_problem(q, k, v, do):
        r = mo.solve_problem(q, k, v, s, cfg.cq, cfg.ck, cfg.topk, cfg.iters)
        if do is not None:
            delta = np.einsum("nd,nd->n", do.astype(np.float64), r.o)
            mo.backward_problem(q, k, v, s, r.aq, r.ak, r.R, min(cfg.cq, len(q)), min(cfg.ck, len(k)),
                                r.lse, delta, do, cfg.dipole)

    t_all = time.perf_counter()
    if not w.causal:
        done = 0
        for h in range(w.Hq):
            g = h * w.Hkv // w.Hq
            one_problem(Q[0, h], K[0, g], V[0, g], None if dO is None else dO[0, h])
            done += 1
            if time.perf_counter() - t_all > budget_s:
                break
        dt = time.perf_counter() - t_all
        value = dt / done * heads * 1e3
        sample = (f"{done} of {heads} whole (batch, query head) problems in {dt:.1f} s, "
                  f"extrapolated linearly in heads")
    else:
        plan = mo.causal_plan(w.N, w.block)
        first = {}
        for pr in plan:
            first.setdefault(pr["level"], pr)
        nseg = {l: sum(1 for pr in plan if pr["level"] == l) for l in first}
        measured, per_level = {}, {}
        for l in sorted(first):
            pr = first[l]
            if measured:
                last = max(measured)
                predicted = measured[last] * pr["kn"] / first[last]["kn"]
                if time.perf_counter() - t_all + predicted > budget_s:
                    break
            q0, qn, k0, kn = pr["q0"], pr["qn"], pr["k0"], pr["kn"]
            t0 = time.perf_counter()
            one_problem(Q[0, 0, q0:q0 + qn], K[0, 0, k0:k0 + kn], V[0, 0, k0:k0 + kn],
                        None if dO is None else dO[0, 0, q0:q0 + qn])
            measured[l] = time.perf_counter() - t0
        lmax = max(measured)
        for l in first:
            per_level[l] = measured[l] if l in measured else measured[lmax] * first[l]["kn"] / first[lmax]["kn"]
        nb = -(-w.N // w.block)
        nloc = min(4, nb)
        t0 = time.perf_counter()
        span = nloc * w.block
        lo, ll = mo.local_causal(Q[0, 0, :span], K[0, 0, :span], V[0, 0, :span], s, w.block)
        if dO is not None:
            delta = np.einsum("nd,nd->n", dO[0, 0, :span].astype(np.float64), lo)
            mo.local_backward(Q[0, 0, :span], K[0, 0, :span], V[0, 0, :span], s, w.block, ll, delta,
                              dO[0, 0, :span])
        t_loc = (time.perf_counter() - t0) * nb / nloc
        per_head = sum(per_level[l] * nseg[l] for l in first) + t_loc
        value = per_head * heads * 1e3
        dt = time.perf_counter() - t_all
        sample = (f"head 0: the first segment of levels {sorted(measured)} timed "
                  f"({', '.join(f'{measured[l]:.2f} s' for l in sorted(measured))}), "
                  f"levels {sorted(set(first) - set(measured))} extrapolated linearly in span, "
                  f"{nloc} of {nb} local blocks timed; {dt:.1f} s of oracle work, scaled by segment "
                  f"counts and {heads} (batch, query head) pairs"
                  + ("; forward + backward" if dO is not None else ""))
    return {"value": round(value, 1), "unit": "ms/layer", "cores": int(_blas_threads()), "kind": "oracle",
            "sample": sample + f"; host os.cpu_count()={os.cpu_count()}"}


def kernel_roofline(w, M, st, rows, step, steps, torch):
    """Per-kernel HIP-event timing (a separate pass of `steps` steps) and the
    roofline of the kernel with the most time per step."""
    M.timing_reset()
    M.timing_enable(True)
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    kt = M.timing_read()
    M.timing_enable(False)
    models = kernel_models(w, M, st, rows)
    # per-level launches (name_L<l>) are summed under their kernel's name
    agg, levels = {}, {}
    for name, (tot, n) in kt.items():
        base = re.sub(r"_L\d+$", "", name)
        a = agg.setdefault(base, [0.0, 0])
        a[0] += tot
        a[1] += n
        if base != name:
            levels[name] = {"ms_per_launch": tot / n, "launches_per_step": n / steps}
    per_kernel = {}
    for name, (tot, n) in agg.items():
        per_kernel[name] = {"ms_per_launch": tot / n, "launches_per_step": n / steps,
                            "ms_per_step": tot / steps}
    dom = max(per_kernel, key=lambda k: per_kernel[k]["ms_per_step"])
    launches = per_kernel[dom]["launches_per_step"]
    fl, by, bound = models.get(dom, (0.0, 0.0, "hbm"))
    avg_s = per_kernel[dom]["ms_per_launch"] / 1e3
    if bound == "mfma":
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        achieved = fl / launches / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None}
    else:
        achieved = by / launches / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None}
    roof["traffic"] = measured_traffic(w, dom)
    roof["kernel"] = dom
    roof["algorithmic_per_launch"] = {"flops": fl / launches, "bytes": by / launches}
    roof["avg_launch_ms"] = round(avg_s * 1e3, 4)
    kernels = {k: {kk: round(vv, 5) for kk, vv in v.items()} for k, v in per_kernel.items()}
    lev = {k: {kk: round(vv, 5) for kk, vv in v.items()} for k, v in levels.items()}
    return roof, kernels, lev


def run_workload(name, args, torch, M, synth, steps, warmup, headline):
    """Time one workload; returns the figures of its JSON entry."""
    w = synth.WORKLOADS[name]
    log(f"{name} ({w.name}): generating inputs")
    x = synth.make_inputs(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    Q, K, V = (torch.from_numpy(x[k]).to(tdt).cuda() for k in ("Q", "K", "V"))
    cfg = M.make_cfg(w.C, w.iters, w.topk, w.causal, w.block)
    rows = M.plan(w.N, cfg)
    O, lse, st = M.museattn_fwd(Q, K, V, cfg)
    ws = torch.empty(M.layout(w.B, w.Hq, w.Hkv, w.N, w.D, M._dt(Q), cfg)["ws_bytes"], dtype=torch.uint8,
                     device="cuda")
    dO = bws = grads = None
    if w.backward:
        dO = torch.from_numpy(x["dO"]).to(tdt).cuda()
        bws = torch.empty(M.bwd_ws_size(w.B, w.Hq, w.Hkv, w.N, w.D, M._dt(Q), cfg), dtype=torch.uint8,
                          device="cuda")
        grads = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))

    def step():
        M.museattn_fwd(Q, K, V, cfg, state=st, ws=ws, out=(O, lse))
        if w.backward:
            M.museattn_bwd(Q, K, V, O, lse, dO, cfg, st, ws=bws, out=grads)

    for _ in range(warmup):
        step()
    log(f"{name}: timing {steps} steps")
    ms, wall = time_steps(step, steps, torch)
    eff = exact_flops(w) / (ms / 1e3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    res = {"workload": w.name, "ms": round(ms, 4), "ms_mean_wall": round(wall, 4),
           "effective_tflops": round(eff, 2), "effective_pct_of_mfma_peak": round(100 * eff / peak, 2),
           "step": "museattn_fwd + museattn_bwd" if w.backward else "museattn_fwd"}
    if headline and not args.no_kernel_timing:
        log(f"{name}: per-kernel timing pass")
        res["roofline"], res["kernels"], res["levels"] = kernel_roofline(w, M, st, rows, step, steps, torch)
    if not args.no_exact:
        log(f"{name}: exact attention (SDPA) and RSE")
        ex_ms = exact_attention_ms(Q, K, V, w, max(3, steps // 2), torch)
        res["exact_attention_same_gpu"] = {"impl": "torch.nn.functional.scaled_dot_product_attention",
                                           "ms": round(ex_ms, 4),
                                           "tflops": round(exact_flops(w) / ex_ms / 1e9, 1),
                                           "speedup_muse_vs_exact": round(ex_ms / ms, 3)}
        rse, rse_row = rse_vs_exact(Q, K, V, O, w, torch)
        res["rse_vs_exact"] = round(rse, 5)
        res["rse_row_mean"] = round(rse_row, 5)
        # the same forward with the exact exponential tilt in place of the dipole
        xcfg = M.make_cfg(w.C, w.iters, w.topk, w.causal, w.block, tilt="exact")
        Ox, lx, stx = M.museattn_fwd(Q, K, V, xcfg)
        wsx = torch.empty(M.layout(w.B, w.Hq, w.Hkv, w.N, w.D, M._dt(Q), xcfg)["ws_bytes"], dtype=torch.uint8,
                          device="cuda")

        def fx():
            M.museattn_fwd(Q, K, V, xcfg, state=stx, ws=wsx, out=(Ox, lx))
        fx()
        x_ms = time_steps(fx, max(3, min(steps // 4, 10)), torch)[0]
        x_rse, x_row = rse_vs_exact(Q, K, V, Ox, w, torch)
        res["exact_tilt"] = {"impl": "museattn_fwd with the exact exponential tilt (forward only)",
                             "ms": round(x_ms, 4), "rse_vs_exact": round(x_rse, 5), "rse_row_mean": round(x_row, 5)}
        del Ox, lx, stx, wsx
        if w.causal and not args.no_blocks:
            # the causal scheme on spatial blocks with accumulated summaries:
            # coarse query clusters (the block's queries in groups of about
            # 64), the workload's key clusters and k1, k2 blocks per cluster
            cq = max(1, w.block // 64)
            bcfg = M.make_cfg(cq, w.iters, w.topk, True, w.block, ck=w.C, blocks=True, topk2=BLOCKS_K2)
            Ob, lb, stb = M.museattn_fwd(Q, K, V, bcfg)
            wsb = torch.empty(M.layout(w.B, w.Hq, w.Hkv, w.N, w.D, M._dt(Q), bcfg)["ws_bytes"],
                              dtype=torch.uint8, device="cuda")

            def fb():
                M.museattn_fwd(Q, K, V, bcfg, state=stb, ws=wsb, out=(Ob, lb))
            fb()
            b_ms = time_steps(fb, max(3, min(steps // 4, 10)), torch)[0]
            b_rse, b_row = rse_vs_exact(Q, K, V, Ob, w, torch)
            res["spatial_blocks"] = {
                "impl": "museattn_fwd, causal spatial blocks with accumulated summaries and two-level "
                        "retrieval (exact tilt; forward only)",
                "query_clusters": cq, "key_clusters": w.C, "k1": w.topk, "k2": BLOCKS_K2,
                "ms": round(b_ms, 4), "rse_vs_exact": round(b_rse, 5), "rse_row_mean": round(b_row, 5)}
            del Ob, lb, stb, wsb
        if headline:
            # the build's own exact attention: every cluster retrieved (forward only)
            own_ms, O_own = own_exact_ms(Q, K, V, w, M, max(2, min(steps // 4, 5)), torch)
            res["exact_attention_own_kernels"] = {
                "impl": "museattn_fwd with k1 = C (all key clusters retrieved; forward only, clustering included)",
                "ms": round(own_ms, 4), "rse_vs_exact": float(f"{rse_vs_exact(Q, K, V, O_own, w, torch)[0]:.3g}")}
            del O_own
    del Q, K, V, O, lse, st, ws, dO, bws, grads
    gc.collect()
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        log(f"{name}: oracle on the host (budget {args.cpu_budget:.0f} s)")
        res["cpu_baseline"] = cpu_baseline(w, x, args.cpu_budget)
    del x
    gc.collect()
    return w, res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    from clustered_approximate_softmax_amd import muse as M
    from clustered_approximate_softmax_amd import synth

    M.lib()   # fail loudly before any work when the HIP library is missing
    w, head = run_workload(args.config, args, torch, M, synth, args.steps, args.warmup, True)
    out = {
        "metric": METRIC, "value": head["ms"], "unit": "ms/layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms"],
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian-mixture Q/K, normal V)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "D": w.D,
                   "clusters": w.C, "lloyd_iters": w.iters, "topk": w.topk, "causal": w.causal,
                   "local_block": w.block, "rope": w.rope, "step": head["step"]},
        "timing": "median of the timed steps by HIP events around each step; ms_mean_wall is the "
                  "host-clock mean over the synchronised region",
        "ms_mean_wall": head["ms_mean_wall"],
        "effective_tflops": head["effective_tflops"],
        "effective_pct_of_mfma_peak": head["effective_pct_of_mfma_peak"],
    }
    for k in ("roofline", "kernels", "levels", "exact_attention_same_gpu", "rse_vs_exact", "rse_row_mean",
              "exact_tilt", "spatial_blocks", "exact_attention_own_kernels", "cpu_baseline"):
        if k in head:
            out[k] = head[k]
    if not args.no_sweep:
        sweep = {}
        for name in SWEEP:
            if name == args.config:
                continue
            ww, r = run_workload(name, args, torch, M, synth, args.sweep_steps, 2, False)
            sweep[name] = r
        out["sweep"] = sweep
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").normal_()
        bbuf = torch.empty_like(a)
        for _ in range(3):
            bbuf.copy_(a)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n * 4
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
