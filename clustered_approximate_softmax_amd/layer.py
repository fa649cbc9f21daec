"""MuSe as a drop-in attention core for PyTorch training.

The pages present MuSe as a replacement for softmax attention that needs
only hyperparameters, no architectural change (newx.sg page, Abstract;
gist.science page, Technical Summary, Key Contributions, Drop-in
Compatibility).  This module wires the C ABI into torch autograd:

* ``MuseAttnFunction``: forward = museattn_fwd, backward = museattn_bwd with
  the forward's clustering held fixed (the saved ``state``);
* ``muse_attention``: the functional form, with an optional warm start of
  the k-means from an earlier call's centroids;
* ``MuseAttention``: a module that replaces ``scaled_dot_product_attention``
  in a layer and warm-starts each training step's clustering from the
  previous step's centroids (queries and keys move little between steps,
  so fewer Lloyd iterations reach the same clustering quality).

Argument marshalling and autograd glue only: every step of the attention
runs in the HIP kernels of libmuse.so.
"""
from __future__ import annotations

from . import muse as M


def _torch():
    import torch
    return torch


def _new_state(q, k, cfg):
    torch = _torch()
    B, Hq, N, D = q.shape
    Hkv = k.shape[1]
    lay = M.layout(B, Hq, Hkv, N, D, M._dt(q), cfg)
    buf = torch.empty(lay["state_bytes"], dtype=torch.uint8, device=q.device)
    return M.State(buf, lay, B, Hq, Hkv, N, D)


def _seed_centroids(st, prev):
    """Copy the query and key centroids of an earlier state into st (same
    layout), for a warm-started k-means; False when the layouts differ."""
    if prev is None or prev.lay != st.lay:
        return False
    P, C, D = st.lay["P"], st.lay["C"], st.D
    for name, heads in (("q_cent", st.B * st.Hq), ("k_cent", st.B * st.Hkv)):
        off = st.lay[name]
        n = heads * P * C * D * 4
        st.buf[off:off + n].copy_(prev.buf[off:off + n])
    return True


class MuseAttnFunction:
    """torch.autograd.Function over museattn_fwd / museattn_bwd (built lazily
    so that importing this module does not import torch)."""

    _cls = None

    @classmethod
    def get(cls):
        if cls._cls is not None:
            return cls._cls
        torch = _torch()

        class _Fn(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, cfg, prev, box):
                st = _new_state(q, k, cfg)
                warm = cfg.init_mode == 1 and _seed_centroids(st, prev)
                run = cfg if warm else M.muse_cfg(cfg.cq, cfg.ck, cfg.iters, cfg.topk, cfg.block, cfg.causal,
                                                  cfg.dipole, 0, cfg.scale, cfg.topk2)
                O, lse, st = M.museattn_fwd(q, k, v, run, state=st)
                ctx.save_for_backward(q, k, v, O, lse)
                ctx.state = st
                ctx.cfg = run
                box["state"] = st
                box["warm"] = warm
                return O

            @staticmethod
            def backward(ctx, dO):
                q, k, v, O, lse = ctx.saved_tensors
                dQ, dK, dV = M.museattn_bwd(q, k, v, O, lse, dO.contiguous(), ctx.cfg, ctx.state)
                return dQ, dK, dV, None, None, None

        cls._cls = _Fn
        return _Fn


def muse_attention(q, k, v, cfg: "M.muse_cfg", prev_state=None):
    """MuSe attention of q [B, Hq, N, D] over k, v [B, Hkv, N, D]
    (contiguous device tensors, bf16 or fp32), differentiable in q, k and v.
    With cfg.init_mode == 1 and prev_state (the state of an earlier call with
    the same shapes and cfg), the k-means continues from prev_state's
    centroids; otherwise it starts from the default points.  Returns
    (O, state)."""
    box = {}
    O = MuseAttnFunction.get().apply(q.contiguous(), k.contiguous(), v.contiguous(), cfg, prev_state, box)
    st = box["state"]
    st.warm_started = box["warm"]
    return O, st


class MuseAttention:
    """Drop-in attention core: ``attn(q, k, v)`` in place of
    ``F.scaled_dot_product_attention(q, k, v, is_causal=causal)`` (scale
    1/sqrt(D)).  Hyperparameters: query clusters ``C`` (key clusters ``ck``,
    default C), retrieved clusters ``topk``, Lloyd iterations ``iters`` (and
    ``warm_iters`` once a previous step's centroids exist, when
    ``warm_start``), causal flag and local ``block`` size."""

    def __init__(self, C, topk, iters=10, causal=False, block=0, ck=None, dipole=True, warm_start=True,
                 warm_iters=None):
        self.C, self.ck, self.topk, self.iters = C, (C if ck is None else ck), topk, iters
        self.causal, self.block, self.dipole = causal, block, dipole
        self.warm_start = warm_start
        self.warm_iters = iters if warm_iters is None else warm_iters
        self.state = None
        self.last_warm = False

    def __call__(self, q, k, v):
        warm = self.warm_start and self.state is not None
        cfg = M.make_cfg(self.C, self.warm_iters if warm else self.iters, self.topk, self.causal, self.block,
                         self.dipole, ck=self.ck, warm=warm)
        O, st = muse_attention(q, k, v, cfg, self.state if warm else None)
        self.state = st
        self.last_warm = st.warm_started
        return O
