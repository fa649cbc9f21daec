"""Benchmark of the MuSe hot path on one MI355X.

A step is one museattn_fwd call over the whole workload tensor (all batch x
heads, clustering included; input generation excluded), inputs resident in
HBM; for the training workload (--config c5) a step is museattn_fwd followed
by museattn_bwd.  Default workload: acausal bf16, batch 1, 8 heads, N=8192, D=64, 64
query and 64 key clusters, 10 Lloyd iterations, top-4 retrieval.

Prints one JSON line: ms per layer, effective TFLOP/s (exact-attention
FLOPs / time), the roofline of the dominant kernel (algorithmic work per
launch / mean launch time from HIP events on the launch stream), exact
attention timed on the same GPU (torch SDPA, and this library's own
kernels with every cluster retrieved), the approximation error (aggregate
and mean per-row RSE on sampled rows), and the fp64 oracle timed on a
bounded sample on the host cores.
"""
import argparse
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="c2", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-exact", action="store_true")
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


def time_calls(fn, steps, torch):
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def exact_attention_ms(Q, K, V, w, steps, torch):
    """torch SDPA on the same tensors (KV heads repeated for GQA); for the
    training workload forward + backward, restricted to the fused flash /
    memory-efficient kernels (no math fallback)."""
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
    return time_calls(f, steps, torch)


def own_exact_ms(Q, K, V, w, M, steps, torch):
    """The same forward with k1 = C: every key cluster is retrieved, so the
    gathered exact kernels compute plain softmax attention (clustering and
    summaries included).  Returns (ms per call, O)."""
    cfg = M.make_cfg(w.C, w.iters, w.C, w.causal, w.block)
    O, lse, st = M.museattn_fwd(Q, K, V, cfg)
    ws = torch.empty(M.layout(w.B, w.Hq, w.Hkv, w.N, w.D, M._dt(Q), cfg)["ws_bytes"], dtype=torch.uint8,
                     device="cuda")

    def f():
        M.museattn_fwd(Q, K, V, cfg, state=st, ws=ws, out=(O, lse))
    f()
    ms = time_calls(f, steps, torch)
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


def cpu_baseline(w, x, budget_s=25.0):
    """Oracle on a bounded sample: one (batch, KV group) slice, or fewer of
    its problems, extrapolated linearly to the whole layer."""
    from oracle import muse_oracle as mo
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    cfg = mo.MuseConfig(cq=w.C, ck=w.C, iters=w.iters, topk=w.topk, block=w.block, causal=w.causal)
    Q, K, V = x["Q"], x["K"], x["V"]
    heads_done = 0
    t0 = time.perf_counter()
    for h in range(w.Hq):
        kv = h * w.Hkv // w.Hq
        mo.forward_head(Q[0, h], K[0, kv], V[0, kv], cfg)
        heads_done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    per_layer_ms = dt / heads_done * (w.B * w.Hq) * 1e3
    return {"value": round(per_layer_ms, 1), "unit": "ms/layer", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{heads_done} of {w.B * w.Hq} (batch, query head) problems in {dt:.1f} s, "
                      f"extrapolated linearly to the layer; host os.cpu_count()={os.cpu_count()}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    from clustered_approximate_softmax_amd import muse as M
    from clustered_approximate_softmax_amd import synth

    w = synth.WORKLOADS[args.config]
    x = synth.make_inputs(w)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    Q, K, V = (torch.from_numpy(x[k]).to(tdt).cuda() for k in ("Q", "K", "V"))
    cfg = M.make_cfg(w.C, w.iters, w.topk, w.causal, w.block)
    rows = M.plan(w.N, cfg)
    O, lse, st = M.museattn_fwd(Q, K, V, cfg)
    ws = torch.empty(M.layout(w.B, w.Hq, w.Hkv, w.N, w.D, M._dt(Q), cfg)["ws_bytes"], dtype=torch.uint8,
                     device="cuda")
    if w.backward:
        dO = torch.from_numpy(x["dO"]).to(tdt).cuda()
        bws = torch.empty(M.bwd_ws_size(w.B, w.Hq, w.Hkv, w.N, w.D, M._dt(Q), cfg), dtype=torch.uint8,
                          device="cuda")
        grads = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))

    def step():
        M.museattn_fwd(Q, K, V, cfg, state=st, ws=ws, out=(O, lse))
        if w.backward:
            M.museattn_bwd(Q, K, V, O, lse, dO, cfg, st, ws=bws, out=grads)

    for _ in range(args.warmup):
        step()
    ms = time_calls(step, args.steps, torch)

    # per-kernel HIP-event timing on the launch stream (separate pass)
    M.timing_reset()
    M.timing_enable(True)
    for _ in range(args.steps):
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
            levels[name] = {"ms_per_launch": tot / n, "launches_per_step": n / args.steps}
    per_kernel = {}
    for name, (tot, n) in agg.items():
        per_kernel[name] = {"ms_per_launch": tot / n, "launches_per_step": n / args.steps,
                            "ms_per_step": tot / args.steps}
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

    eff = exact_flops(w) / (ms / 1e3) / 1e12
    out = {
        "metric": METRIC, "value": round(ms, 4), "unit": "ms/layer", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian-mixture Q/K, normal V)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "N": w.N, "D": w.D,
                   "clusters": w.C, "lloyd_iters": w.iters, "topk": w.topk, "causal": w.causal,
                   "local_block": w.block},
        "effective_tflops": round(eff, 2),
        "effective_pct_of_mfma_peak": round(100 * eff / (PEAK_BF16_TFLOPS if w.dtype == "bf16"
                                                           else PEAK_F32_TFLOPS), 2),
        "roofline": roof,
        "kernels": {k: {kk: round(vv, 5) for kk, vv in v.items()} for k, v in per_kernel.items()},
        "levels": {k: {kk: round(vv, 5) for kk, vv in v.items()} for k, v in levels.items()},
    }
    if not args.no_exact:
        ex_ms = exact_attention_ms(Q, K, V, w, max(3, args.steps // 2), torch)
        out["exact_attention_same_gpu"] = {"impl": "torch.nn.functional.scaled_dot_product_attention",
                                           "ms": round(ex_ms, 4),
                                           "tflops": round(exact_flops(w) / ex_ms / 1e9, 1),
                                           "speedup_muse_vs_exact": round(ex_ms / ms, 3)}
        rse, rse_row = rse_vs_exact(Q, K, V, O, w, torch)
        out["rse_vs_exact"] = round(rse, 5)
        out["rse_row_mean"] = round(rse_row, 5)
        # the build's own exact attention: every cluster retrieved (forward only)
        own_ms, O_own = own_exact_ms(Q, K, V, w, M, max(2, args.steps // 4), torch)
        out["exact_attention_own_kernels"] = {
            "impl": "museattn_fwd with k1 = C (all key clusters retrieved; forward only, clustering included)",
            "ms": round(own_ms, 4), "rse_vs_exact": float(f"{rse_vs_exact(Q, K, V, O_own, w, torch)[0]:.3g}")}
        del O_own
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device="cuda").normal_()
        bbuf = torch.empty_like(a)
        for _ in range(3):
            bbuf.copy_(a)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = n * 4
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
