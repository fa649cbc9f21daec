"""Host-side checks of the C ABI (no GPU needed): the library loads and
exports every function include/muse.h declares, the problem plan equals the
oracle's causal hierarchy, and argument validation returns error codes
before anything is queued."""
import ctypes

import numpy as np
import pytest

from clustered_approximate_softmax_amd import muse as M
from oracle import muse_oracle as mo


def test_library_exports_every_declared_function():
    L = M.lib()
    names = M.header_functions()
    assert {"musecluster", "musesummarize", "museattn_fwd", "museattn_bwd"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_strerror():
    L = M.lib()
    for code in (0, -1, -2, -3, -4, 7):
        assert len(L.muse_strerror(code)) > 3


@pytest.mark.parametrize("N,B", [(64, 8), (65, 8), (100, 16), (1024, 64), (16384, 512), (65536, 1024),
                                 (30, 64), (1000, 16)])
def test_plan_matches_oracle_hierarchy(N, B):
    got = M.plan(N, M.make_cfg(8, causal=True, block=B))
    want = mo.causal_plan(N, B)
    assert len(got) == len(want)
    for g, w in zip(got, want):
        assert tuple(g) == (w["level"], w["t"], w["k0"], w["kn"], w["q0"], w["qn"])


def test_acausal_plan_is_one_problem():
    got = M.plan(777, M.make_cfg(8))
    assert got.tolist() == [[0, 0, 0, 777, 0, 777]]


def test_layout_sizes():
    cfg = M.make_cfg(64, 10, 4)
    lay = M.layout(1, 8, 8, 8192, 64, M.MUSE_BF16, cfg)
    assert lay["P"] == 1 and lay["L"] == 1 and lay["k1w"] == 4 and lay["Cp32"] == 64
    assert lay["M"] + 8 * 64 * 64 * 64 * 4 <= lay["R"]
    assert lay["state_bytes"] >= lay["R"] + 8 * 64 * 4 * 4
    assert lay["ws_bytes"] >= 8 * 64 * 64 * 64 * 4
    # value columns: one sorted copy per head, rows padded to 8 (acausal: no input-order copy)
    assert lay["Nv"] == 8192 and lay["ws_Vt"] + 8 * 64 * 8192 * 2 <= lay["ws_bytes"]
    odd = M.layout(1, 1, 1, 1001, 64, M.MUSE_BF16, M.make_cfg(16, 3, 2, True, 100))
    assert odd["Nv"] == 1008
    assert odd["ws_Vt"] + (odd["L"] + 1) * 64 * 1008 * 2 <= odd["ws_bytes"]
    c4 = M.layout(1, 32, 8, 65536, 64, M.MUSE_BF16, M.make_cfg(128, 10, 8, True, 1024))
    assert c4["P"] == 63 and c4["L"] == 6


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first


def _fwd(cfg, B=1, Hq=2, Hkv=2, N=256, D=64, dtype=M.MUSE_BF16, ws=1 << 40, st=1 << 40, ptr=FAKE):
    return M.lib().museattn_fwd(ptr, ptr, ptr, dtype, B, Hq, Hkv, N, D, ctypes.byref(cfg), None, None, ptr,
                                ptr, ptr, st, ptr, ws, None)


@pytest.mark.parametrize("kw,cfgkw", [
    (dict(D=32), {}), (dict(D=96), {}), (dict(Hq=3, Hkv=2), {}), (dict(N=0), {}), (dict(B=0), {}),
    (dict(dtype=7), {}), ({}, dict(C=0)), ({}, dict(C=257)), ({}, dict(iters=0)),
    ({}, dict(topk=-1)), ({}, dict(causal=True, block=0)),
])
def test_fwd_rejects_bad_arguments(kw, cfgkw):
    c = dict(C=16, iters=3, topk=1, causal=False, block=0)
    c.update(cfgkw)
    assert _fwd(M.make_cfg(**c), **kw) == -1


def test_fwd_rejects_bad_key_cluster_count_and_nulls():
    for ck in (0, 257):
        assert _fwd(M.make_cfg(16, 3, 1, ck=ck)) == -1
    assert _fwd(M.make_cfg(16, 3, 1), ptr=None) == -1


def test_layout_with_separate_cluster_counts():
    """Per-cluster arrays use max(cq, ck) clusters; the retrieval width
    follows the key clusters."""
    lay = M.layout(1, 2, 1, 4096, 64, M.MUSE_BF16, M.make_cfg(24, 3, 40, ck=80))
    assert lay["C"] == 80 and lay["k1w"] == 40 and lay["Cp32"] == 128
    lay = M.layout(1, 2, 1, 4096, 64, M.MUSE_BF16, M.make_cfg(96, 3, 40, ck=16))
    assert lay["C"] == 96 and lay["k1w"] == 16


def test_fwd_rejects_small_buffers():
    cfg = M.make_cfg(16, 3, 1)
    assert _fwd(cfg, ws=16) == -2
    assert _fwd(cfg, st=16) == -2


def test_cluster_and_summarize_reject_bad_arguments():
    L = M.lib()
    assert L.musecluster(FAKE, 1, 2, 100, 48, 8, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert L.musecluster(FAKE, 1, 2, 100, 64, 300, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert L.musecluster(None, 1, 2, 100, 64, 8, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    # a large problem needs workspace for its chunk partials
    assert L.muse_cluster_ws_size(2, 100000, 64, 1, 64) > 0
    assert L.musecluster(FAKE, 1, 2, 100000, 64, 64, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE, 8, None) == -2
    assert L.musesummarize(FAKE, FAKE, 1, 2, 100, 64, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1


def test_backward_entry_point_exported():
    assert hasattr(M.lib(), "museattn_bwd")


def test_entry_points_reject_misaligned_tensors():
    odd = ctypes.c_void_p(0x1008)   # 8-byte aligned only
    assert _fwd(M.make_cfg(16, 3, 1), ptr=odd) == -1
    L = M.lib()
    assert L.musecluster(odd, 1, 2, 100, 64, 8, 3, None, FAKE, FAKE, FAKE, FAKE, None, 0, None) == -1
    assert L.musesummarize(odd, FAKE, 1, 2, 100, 64, 8, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1


def test_bwd_ws_size_and_null_checks():
    L = M.lib()
    cfg = M.make_cfg(16, 2, 2, True, 64)
    n = L.muse_bwd_ws_size(1, 4, 2, 1000, 64, 1, ctypes.byref(cfg))
    # at least the fp32 gradient accumulators and Delta
    assert n >= (4 * 1000 * 64 + 2 * 2 * 1000 * 64 + 4 * 1000) * 4
    bad = M.make_cfg(16, 2, 2, True, 64)
    assert L.muse_bwd_ws_size(1, 3, 2, 1000, 64, 1, ctypes.byref(bad)) == 0      # Hq % Hkv != 0
    assert L.muse_bwd_ws_size(1, 4, 2, 1000, 96, 1, ctypes.byref(bad)) == 0      # D unsupported
    rc = L.museattn_bwd(None, None, None, None, None, None, 1, 1, 4, 2, 1000, 64, ctypes.byref(cfg),
                        None, 0, None, None, None, None, 0, None)
    assert rc == -1


def test_noalloc_forward_rejects_workspace_beyond_its_array():
    """museattn_fwd_noalloc checks the call's workspace against its fixed
    per-GPU array (64 MiB) before touching the GPU."""
    L = M.lib()
    big = M.make_cfg(32, 10, 0, True, 512)          # 16k causal, batch 4, 8 heads: ~770 MiB
    assert M.layout(4, 8, 8, 16384, 64, M.MUSE_BF16, big)["ws_bytes"] > 64 << 20
    rc = L.museattn_fwd_noalloc(FAKE, FAKE, FAKE, M.MUSE_BF16, 4, 8, 8, 16384, 64, ctypes.byref(big), None, None,
                                FAKE, FAKE, FAKE, 1 << 40, None)
    assert rc == -2
    rc = L.museattn_fwd_noalloc(FAKE, FAKE, FAKE, M.MUSE_BF16, 1, 2, 2, 256, 32, ctypes.byref(big), None, None,
                                FAKE, FAKE, FAKE, 1 << 40, None)
    assert rc == -1


def test_spatial_block_scheme_validation_and_layout():
    """causal = 2 (spatial blocks with accumulated summaries) needs the exact
    tilt, k2 >= 1 when k1 >= 1, at most 4096 blocks and k1w * k2w <= 256;
    its state holds the retrieval of every group and the block starts."""
    L = M.lib()
    ok = M.make_cfg(16, 3, 4, True, 64, ck=32, blocks=True, topk2=3)
    lay = M.layout(1, 4, 2, 1000, 64, M.MUSE_BF16, ok)
    assert lay["P"] == 1 and lay["L"] == 1 and lay["nb"] == 16 and lay["k2w"] == 3 and lay["k1w"] == 4
    assert lay["v4_R2"] >= lay["v4_R1"] + 4 * 16 * 16 * 4 * 4
    assert lay["state_bytes"] >= lay["v4_qb"] + 4 * 16 * 17 * 4
    assert lay["ws_bytes"] >= lay["ws_v4fb"] + 4 * 16 * 16 * lay["Cp32"] * 4
    assert lay["ws_oacc"] == lay["ws_T"]            # the hierarchy's T is not allocated
    for bad, code in ((dict(tilt="dipole"), -3), (dict(topk2=0), -1), (dict(topk2=-1), -1)):
        c = M.make_cfg(16, 3, 4, True, 64, ck=32, blocks=True, topk2=bad.get("topk2", 3))
        if "tilt" in bad:
            c.dipole = 1
        assert L.muse_layout_query(1, 4, 2, 1000, 64, 1, ctypes.byref(c), ctypes.byref(M.muse_layout())) == code
    many = M.make_cfg(16, 3, 4, True, 4, ck=32, blocks=True, topk2=3)        # 5000 blocks
    assert L.muse_layout_query(1, 1, 1, 20000, 64, 1, ctypes.byref(many), ctypes.byref(M.muse_layout())) == -3
    wide = M.make_cfg(16, 3, 32, True, 16, ck=32, blocks=True, topk2=9)     # 32 x 9 > 256 pairs
    assert L.muse_layout_query(1, 1, 1, 1000, 64, 1, ctypes.byref(wide), ctypes.byref(M.muse_layout())) == -3
    # no retrieval: k2 may be 0
    none = M.make_cfg(16, 3, 0, True, 64, ck=32, blocks=True, topk2=0)
    assert L.muse_layout_query(1, 1, 1, 1000, 64, 1, ctypes.byref(none), ctypes.byref(M.muse_layout())) == 0
    # the backward does not cover the scheme
    assert L.museattn_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 4, 2, 1000, 64, ctypes.byref(ok), FAKE,
                          1 << 40, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == -3
