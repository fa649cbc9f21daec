"""Python binding of the MuSe HIP library (include/muse.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libmuse.so.  Tensors are torch CUDA (HIP) tensors; PyTorch is used
for device memory and the current stream.  There is no CPU fallback: a
missing library raises ``MuseLibraryMissing``.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "_build", "libmuse.so")
HEADER = os.path.join(ROOT, "include", "muse.h")

MUSE_F32, MUSE_BF16 = 0, 1
ERRORS = {0: "MUSE_OK", -1: "MUSE_EINVAL", -2: "MUSE_EWORKSPACE", -3: "MUSE_EUNSUPPORTED",
          -4: "MUSE_EHIP"}


class MuseLibraryMissing(RuntimeError):
    pass


class MuseError(RuntimeError):
    def __init__(self, fn, code, detail=""):
        self.code = code
        super().__init__(f"{fn} failed: {ERRORS.get(code, code)} {detail}".strip())


class muse_cfg(ctypes.Structure):
    _fields_ = [("cq", ctypes.c_int32), ("ck", ctypes.c_int32), ("iters", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("block", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("dipole", ctypes.c_int32), ("init_mode", ctypes.c_int32), ("scale", ctypes.c_float),
                ("topk2", ctypes.c_int32)]


LAYOUT_FIELDS = ["P", "L", "C", "k1w", "Cp32", "Nv"]
LAYOUT_OFFS = ["q_labels", "k_labels", "q_perm", "k_perm", "q_offs", "k_offs", "q_cent", "k_cent",
               "mu", "S", "M", "R", "Kp", "Vp", "mu_in", "state_bytes", "ws_T", "ws_oacc", "ws_lacc", "ws_Vt", "ws_part",
               "ws_pcnt", "ws_bytes", "ws_kap", "ws_lz", "ws_fb"]
LAYOUT_V4_FIELDS = ["nb", "k2w"]
LAYOUT_V4_OFFS = ["v4_R1", "v4_R2", "v4_kb", "v4_qb", "ws_v4pz", "ws_v4pk", "ws_v4pu", "ws_v4kap", "ws_v4T",
                  "ws_v4fb"]


class muse_layout(ctypes.Structure):
    _fields_ = ([(n, ctypes.c_int64) for n in LAYOUT_FIELDS] + [(n, ctypes.c_size_t) for n in LAYOUT_OFFS]
                + [(n, ctypes.c_int64) for n in LAYOUT_V4_FIELDS] + [(n, ctypes.c_size_t) for n in LAYOUT_V4_OFFS])


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def lib():
    """Load libmuse.so (built in-tree by build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise MuseLibraryMissing(f"{LIB_PATH} is not built; run clustered_approximate_softmax_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    L.muse_strerror.restype = ctypes.c_char_p
    L.muse_strerror.argtypes = [ctypes.c_int]
    L.muse_last_hip_error.restype = ctypes.c_char_p
    L.muse_plan.argtypes = [_I64, ctypes.POINTER(muse_cfg), ctypes.POINTER(ctypes.c_int32), _I64,
                            ctypes.POINTER(ctypes.c_int64)]
    L.muse_layout_query.argtypes = [_I64, _I64, _I64, _I64, _I64, ctypes.c_int, ctypes.POINTER(muse_cfg),
                                    ctypes.POINTER(muse_layout)]
    L.muse_cluster_ws_size.restype = ctypes.c_size_t
    L.muse_cluster_ws_size.argtypes = [_I64, _I64, _I64, ctypes.c_int, _I32]
    L.musecluster.argtypes = [_P, ctypes.c_int, _I64, _I64, _I64, _I32, _I32, _P, _P, _P, _P, _P, _P,
                              ctypes.c_size_t, _P]
    L.musesummarize.argtypes = [_P, _P, ctypes.c_int, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P]
    L.museattn_fwd.argtypes = [_P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _I64, _I64,
                               ctypes.POINTER(muse_cfg), _P, _P, _P, _P, _P, ctypes.c_size_t, _P,
                               ctypes.c_size_t, _P]
    L.museattn_fwd_noalloc.argtypes = [_P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _I64, _I64,
                                       ctypes.POINTER(muse_cfg), _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    L.muse_bwd_ws_size.restype = ctypes.c_size_t
    L.muse_bwd_ws_size.argtypes = [_I64, _I64, _I64, _I64, _I64, ctypes.c_int, ctypes.POINTER(muse_cfg)]
    L.museattn_bwd.argtypes = [_P, _P, _P, _P, _P, _P, ctypes.c_int, _I64, _I64, _I64, _I64, _I64,
                               ctypes.POINTER(muse_cfg), _P, ctypes.c_size_t, _P, _P, _P, _P,
                               ctypes.c_size_t, _P]
    L.muse_timing_get.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                  ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    _lib = L
    return L


def header_functions():
    """Names of the functions declared in include/muse.h."""
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(muse\w*)\s*\(", txt)))


def _check(fn, rc):
    if rc != 0:
        detail = lib().muse_last_hip_error().decode() if rc == -4 else ""
        raise MuseError(fn, rc, detail)


TILT = {"monopole": 0, "dipole": 1, "exact": 2}


def make_cfg(C, iters=10, topk=0, causal=False, block=0, dipole=True, scale=0.0, ck=None, warm=False,
             tilt=None, blocks=False, topk2=0):
    """C query clusters (and key clusters unless ck is given); warm: the
    k-means continues from the centroids of the state passed to the call;
    tilt: "monopole", "dipole" or "exact" (overrides dipole); blocks: the
    causal scheme on spatial blocks with accumulated summaries (causal = 2,
    exact tilt, topk2 blocks inside each of the topk retrieved clusters)."""
    if blocks:
        tilt = "exact"
    mode = TILT[tilt] if tilt is not None else int(bool(dipole))
    cz = 2 if blocks else int(bool(causal))
    return muse_cfg(int(C), int(C if ck is None else ck), int(iters), int(topk), int(block),
                    cz, mode, int(bool(warm)), float(scale), int(topk2))


def plan(N, cfg: muse_cfg):
    cnt = ctypes.c_int64(0)
    _check("muse_plan", lib().muse_plan(N, ctypes.byref(cfg), None, 0, ctypes.byref(cnt)))
    out = np.zeros((max(cnt.value, 1), 6), np.int32)
    _check("muse_plan", lib().muse_plan(N, ctypes.byref(cfg), out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                        cnt.value, ctypes.byref(cnt)))
    return out[: cnt.value]


def layout(B, Hq, Hkv, N, D, dtype, cfg: muse_cfg) -> dict:
    lay = muse_layout()
    _check("muse_layout_query", lib().muse_layout_query(B, Hq, Hkv, N, D, dtype, ctypes.byref(cfg),
                                                        ctypes.byref(lay)))
    out = {n: int(getattr(lay, n)) for n, _ in muse_layout._fields_}
    out.update(cq=int(cfg.cq), ck=int(cfg.ck))
    return out


# ---------------------------------------------------------------------------
# torch-facing wrappers
# ---------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dt(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MUSE_BF16
    if t.dtype == torch.float32:
        return MUSE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev_check(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("tensors must be contiguous device tensors")


def musecluster(X, C, iters, init_idx=None):
    """X [G, n, D] -> assign [G,n] int32, centroids [G,C,D] f32, perm [G,n], offs [G,C+1]."""
    torch = _torch()
    _dev_check(X, init_idx)
    G, n, D = X.shape
    dev = X.device
    assign = torch.empty((G, n), dtype=torch.int32, device=dev)
    cent = torch.empty((G, C, D), dtype=torch.float32, device=dev)
    perm = torch.empty((G, n), dtype=torch.int32, device=dev)
    offs = torch.empty((G, C + 1), dtype=torch.int32, device=dev)
    wsb = lib().muse_cluster_ws_size(G, n, D, _dt(X), C)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    rc = lib().musecluster(_ptr(X), _dt(X), G, n, D, C, iters, _ptr(init_idx), _ptr(assign), _ptr(cent),
                           _ptr(perm), _ptr(offs), _ptr(ws), ws.numel(), _stream())
    _check("musecluster", rc)
    return assign, cent, perm, offs


def musesummarize(K, V, assign, C):
    """K, V [G, n, D], assign [G, n] -> perm, offs, mu [G,C,D], S [G,C,D], M [G,D,C,D]."""
    torch = _torch()
    _dev_check(K, V, assign)
    G, n, D = K.shape
    dev = K.device
    perm = torch.empty((G, n), dtype=torch.int32, device=dev)
    offs = torch.empty((G, C + 1), dtype=torch.int32, device=dev)
    mu = torch.empty((G, C, D), dtype=torch.float32, device=dev)
    S = torch.empty((G, C, D), dtype=torch.float32, device=dev)
    M = torch.empty((G, D, C, D), dtype=torch.float32, device=dev)
    rc = lib().musesummarize(_ptr(K), _ptr(V), _dt(K), G, n, D, C, _ptr(assign), _ptr(perm), _ptr(offs),
                             _ptr(mu), _ptr(S), _ptr(M), _stream())
    _check("musesummarize", rc)
    return perm, offs, mu, S, M


@dataclass
class State:
    """The state buffer written by museattn_fwd, with typed views."""

    buf: object
    lay: dict
    B: int
    Hq: int
    Hkv: int
    N: int
    D: int

    def _view(self, name, dtype, shape):
        torch = _torch()
        off = self.lay[name]
        nbytes = int(np.prod(shape)) * 4
        return self.buf[off:off + nbytes].view(dtype).view(*shape)

    def field(self, name):
        torch = _torch()
        P, L, C, k1w = self.lay["P"], self.lay["L"], self.lay["C"], self.lay["k1w"]
        BHq, BHk, N, D = self.B * self.Hq, self.B * self.Hkv, self.N, self.D
        i32, f32 = torch.int32, torch.float32
        shapes = {
            "q_labels": (i32, (L, BHq, N)), "k_labels": (i32, (L, BHk, N)),
            "q_perm": (i32, (L, BHq, N)), "k_perm": (i32, (L, BHk, N)),
            "q_offs": (i32, (BHq, P, C + 1)), "k_offs": (i32, (BHk, P, C + 1)),
            "q_cent": (f32, (BHq, P, C, D)), "k_cent": (f32, (BHk, P, C, D)),
            "mu": (f32, (BHk, P, C, D)), "S": (f32, (BHk, P, C, D)),
            "M": (f32, (BHk, P, D, C, D)), "R": (i32, (BHq, P, C, k1w)),
        }
        nb, k2w = self.lay["nb"], self.lay["k2w"]
        if nb:
            Cq, Ck = self.lay["cq"], self.lay["ck"]
            shapes.update({
                "v4_R1": (i32, (BHq, Cq, nb, k1w)), "v4_R2": (i32, (BHq, Cq, nb, k1w, k2w)),
                "v4_kb": (i32, (BHk, Ck, nb + 1)), "v4_qb": (i32, (BHq, Cq, nb + 1)),
            })
        dt, shp = shapes[name]
        return self._view(name, dt, shp)


def museattn_fwd(Q, K, V, cfg: muse_cfg, init_q=None, init_k=None, state=None, ws=None, out=None):
    """Q [B,Hq,N,D], K/V [B,Hkv,N,D] -> (O, lse, State).  Buffers may be reused
    across calls by passing state / ws / out=(O, lse)."""
    torch = _torch()
    _dev_check(Q, K, V, init_q, init_k)
    B, Hq, N, D = Q.shape
    Hkv = K.shape[1]
    dt = _dt(Q)
    lay = layout(B, Hq, Hkv, N, D, dt, cfg)
    dev = Q.device
    if state is None:
        state = State(torch.empty(lay["state_bytes"], dtype=torch.uint8, device=dev), lay, B, Hq, Hkv, N, D)
    if ws is None:
        ws = torch.empty(lay["ws_bytes"], dtype=torch.uint8, device=dev)
    if out is None:
        O = torch.empty_like(Q)
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    else:
        O, lse = out
    rc = lib().museattn_fwd(_ptr(Q), _ptr(K), _ptr(V), dt, B, Hq, Hkv, N, D, ctypes.byref(cfg), _ptr(init_q),
                            _ptr(init_k), _ptr(O), _ptr(lse), _ptr(state.buf), state.buf.numel(), _ptr(ws),
                            ws.numel(), _stream())
    _check("museattn_fwd", rc)
    return O, lse, state


def museattn_fwd_noalloc(Q, K, V, cfg: muse_cfg, state: "State", out, init_q=None, init_k=None):
    """museattn_fwd on the library's own per-GPU workspace: state and
    out=(O, lse) are given by the caller, nothing is allocated."""
    _dev_check(Q, K, V, init_q, init_k)
    B, Hq, N, D = Q.shape
    Hkv = K.shape[1]
    O, lse = out
    rc = lib().museattn_fwd_noalloc(_ptr(Q), _ptr(K), _ptr(V), _dt(Q), B, Hq, Hkv, N, D, ctypes.byref(cfg),
                                    _ptr(init_q), _ptr(init_k), _ptr(O), _ptr(lse), _ptr(state.buf),
                                    state.buf.numel(), _stream())
    _check("museattn_fwd_noalloc", rc)
    return O, lse, state


def bwd_ws_size(B, Hq, Hkv, N, D, dtype, cfg: muse_cfg) -> int:
    n = lib().muse_bwd_ws_size(B, Hq, Hkv, N, D, dtype, ctypes.byref(cfg))
    if n == 0:
        raise MuseError("muse_bwd_ws_size", -1, "invalid shape or parameters")
    return n


def museattn_bwd(Q, K, V, O, lse, dO, cfg: muse_cfg, state: State, ws=None, out=None):
    """Gradients (dQ, dK, dV) of museattn_fwd with the clustering in `state`
    held fixed.  ws (uint8, >= bwd_ws_size bytes) and out=(dQ, dK, dV) may be
    passed in to reuse buffers."""
    torch = _torch()
    _dev_check(Q, K, V, O, lse, dO)
    B, Hq, N, D = Q.shape
    Hkv = K.shape[1]
    dt = _dt(Q)
    wsb = bwd_ws_size(B, Hq, Hkv, N, D, dt, cfg)
    if ws is None or ws.numel() < wsb:
        ws = torch.empty(wsb, dtype=torch.uint8, device=Q.device)
    if out is None:
        dQ, dK, dV = torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V)
    else:
        dQ, dK, dV = out
    rc = lib().museattn_bwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(lse), _ptr(dO), dt, B, Hq, Hkv, N, D,
                            ctypes.byref(cfg), _ptr(state.buf), state.buf.numel(), _ptr(dQ), _ptr(dK),
                            _ptr(dV), _ptr(ws), ws.numel(), _stream())
    _check("museattn_bwd", rc)
    return dQ, dK, dV


# ---------------------------------------------------------------------------
# per-kernel timing (HIP events recorded by the library on its launch stream)
# ---------------------------------------------------------------------------
def timing_enable(on=True):
    lib().muse_timing_enable(1 if on else 0)


def timing_reset():
    lib().muse_timing_reset()


def timing_read():
    L = lib()
    L.muse_timing_collect()
    out = {}
    i = 0
    while True:
        name = ctypes.c_char_p()
        ms = ctypes.c_double()
        n = ctypes.c_int64()
        if L.muse_timing_get(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(n)) != 0:
            break
        out[name.value.decode()] = (ms.value, n.value)
        i += 1
    return out
