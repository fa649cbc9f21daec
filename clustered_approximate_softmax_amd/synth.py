"""Seeded synthetic inputs for MuSe workloads.

This module only draws inputs: it holds none of the method's arithmetic, and
both the HIP path and the fp64 oracle consume what it returns.

The pages measure on real attention inputs (code, science documents, book
texts, Llama 3 activations) that are not available here; a per-head Gaussian
mixture stands in for them: component centres z / sqrt(8) with
z ~ N(0, I_D), equal-weight labels, points centre + 0.3 eps, eps ~ N(0, I_D),
queries and keys from independent mixtures, values and upstream gradients
N(0, 1).  Configurations that use Llama shapes get rotary position
embeddings (base 500000, rotate-half pairing, positions 0..N-1) applied in
float64 before the cast.

Seeds: numpy SeedSequence(20260 + config number) spawned into nine streams
in the fixed order Q centres, Q labels, Q noise, K centres, K labels,
K noise, V, dO, init.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

STREAMS = ("qc", "ql", "qn", "kc", "kl", "kn", "v", "do", "init")


@dataclass(frozen=True)
class Workload:
    """One benchmark shape (batch, heads, length, dim, dtype, MuSe params)."""

    name: str
    number: int
    B: int
    Hq: int
    Hkv: int
    N: int
    D: int
    dtype: str            # "f32" or "bf16"
    C: int
    iters: int
    topk: int
    causal: bool
    block: int
    comps: int
    rope: bool
    backward: bool
    seeded_init: bool

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "c1": Workload("acausal-f32-N1024-H1-D64-C16", 1, 1, 1, 1, 1024, 64, "f32", 16, 10, 0,
                   False, 0, 16, False, False, True),
    "c2": Workload("acausal-bf16-N8192-H8-D64-C64-top4", 2, 1, 8, 8, 8192, 64, "bf16", 64, 10, 4,
                   False, 0, 64, False, False, False),
    "c3": Workload("causal-bf16-B4-N16384-H8-D64-local512-C32", 3, 4, 8, 8, 16384, 64, "bf16", 32,
                   10, 0, True, 512, 64, False, False, False),
    "c4": Workload("causal-bf16-N65536-Hq32-Hkv8-D64-rope-local1024-C128-top8", 4, 1, 32, 8, 65536,
                   64, "bf16", 128, 10, 8, True, 1024, 64, True, False, False),
    "c5": Workload("causal-bf16-N65536-Hq32-Hkv8-D128-rope-local1024-C128-top8-fwdbwd", 5, 1, 32, 8,
                   65536, 128, "bf16", 128, 10, 8, True, 1024, 64, True, True, False),
}


def streams(number: int) -> dict:
    ss = np.random.SeedSequence(20260 + number)
    return {name: np.random.Generator(np.random.PCG64(child))
            for name, child in zip(STREAMS, ss.spawn(len(STREAMS)))}


def mixture(rc, rl, rn, B, H, N, D, comps, sigma=0.3):
    """[B, H, N, D] float64 points of an independent mixture per (b, h)."""
    centres = rc.standard_normal((B, H, comps, D)) / np.sqrt(8.0)
    labels = rl.integers(0, comps, size=(B, H, N))
    x = np.take_along_axis(centres, labels[..., None], axis=2)
    x += sigma * rn.standard_normal((B, H, N, D))
    return x


def rope(x, base=500000.0):
    """Rotary embedding, rotate-half pairing (i, i + D/2), positions 0..N-1."""
    N, D = x.shape[-2], x.shape[-1]
    half = D // 2
    inv = base ** (-2.0 * np.arange(half) / D)
    ang = np.arange(N)[:, None] * inv[None, :]
    cos, sin = np.cos(ang), np.sin(ang)
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * cos - b * sin, a * sin + b * cos], axis=-1)


def to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 to the storage type and return it as float32 holding
    exactly the stored values (bf16: round to nearest even on the top 16
    bits of the float32 image)."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return f
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return rounded.astype(np.uint32).view(np.float32)


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exactly bf16."""
    return (np.ascontiguousarray(x32, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def make_inputs(w: Workload, with_do: bool = None, heads=None):
    """Q [B,Hq,N,D], K/V [B,Hkv,N,D] (and dO) as float32 arrays holding the
    exact values of the storage dtype, plus the generator of the init stream.
    """
    r = streams(w.number)
    Q = mixture(r["qc"], r["ql"], r["qn"], w.B, w.Hq, w.N, w.D, w.comps)
    K = mixture(r["kc"], r["kl"], r["kn"], w.B, w.Hkv, w.N, w.D, w.comps)
    if w.rope:
        Q = rope(Q)
        K = rope(K)
    V = r["v"].standard_normal((w.B, w.Hkv, w.N, w.D))
    out = dict(Q=to_dtype(Q, w.dtype), K=to_dtype(K, w.dtype), V=to_dtype(V, w.dtype))
    del Q, K, V
    if with_do if with_do is not None else w.backward:
        out["dO"] = to_dtype(r["do"].standard_normal((w.B, w.Hq, w.N, w.D)), w.dtype)
    out["init_rng"] = r["init"]
    return out


def draw_inits(rng, sizes, C):
    """For each problem size n: C distinct indices from range(n) (the first
    min(C, n) are used), drawn with Generator.choice(n, min(C,n), replace=False)
    and padded with -1.  Returns int32 [len(sizes), C]."""
    out = np.full((len(sizes), C), -1, np.int32)
    for p, n in enumerate(sizes):
        c = min(C, n)
        out[p, :c] = rng.choice(n, c, replace=False)
    return out
