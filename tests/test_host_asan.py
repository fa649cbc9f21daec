"""Host code of the C ABI under AddressSanitizer (CPU only, no GPU needed).

capi.hip is rebuilt with the sanitizer on its host side only (the device
code is unchanged) and linked with the in-tree objects of the other sources.
A child process then runs every host-only path of the ABI under the
sanitizer runtime: the problem plan and the state/workspace layout for many
shapes and configurations (causal hierarchy, spatial blocks, separate
cluster counts, ragged and tiny sizes, up to 2^20 rows), and the argument
checks of every entry point that returns before anything is queued.  Any
out-of-bounds access or use of freed memory in that code aborts the child
with a sanitizer report.  A tiny program with a planted heap overflow checks
first that the sanitizer runtime reports one here."""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "clustered_approximate_softmax_amd")
HIPCC = "/opt/rocm/bin/hipcc"
CLANGXX = "/opt/rocm/llvm/bin/clang++"


def _asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _objects():
    return sorted(o for o in glob.glob(os.path.join(PKG, "_build", "*.o")) if os.path.basename(o) != "capi.o")


pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) and _asan_runtime() and len(_objects()) >= 6),
                                reason="needs hipcc, the clang sanitizer runtime and the in-tree build objects")

HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def _env():
    env = dict(os.environ)
    env["LD_PRELOAD"] = _asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0:exitcode=23"
    return env


def test_sanitizer_reports_a_planted_overflow(tmp_path):
    src = tmp_path / "overflow.cpp"
    src.write_text("#include <cstdlib>\nint main(int c, char**) { int* p = (int*)malloc(8 * sizeof(int));"
                   " int v = p[8 + c]; free(p); return v; }\n")
    exe = tmp_path / "overflow"
    subprocess.run([CLANGXX, "-O0", "-g", "-fsanitize=address", str(src), "-o", str(exe)], check=True,
                   capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env={**os.environ,
                                                                      "ASAN_OPTIONS": "exitcode=23"})
    assert r.returncode == 23 and "heap-buffer-overflow" in r.stderr


CHILD = textwrap.dedent(r"""
    import ctypes, sys
    sys.path.insert(0, ROOT)
    from clustered_approximate_softmax_amd import muse as M
    M.LIB_PATH = LIB
    L = M.lib()
    FAKE = ctypes.c_void_p(0x1000)
    n = 0
    # problem plans: causal hierarchies up to the level limit, ragged sizes
    for N in (1, 2, 7, 63, 64, 65, 1000, 4097, 65536, 1 << 20):
        for blk in (1, 3, 16, 64, 1000, 1024):
            for causal in (0, 1, 2):
                cfg = M.make_cfg(8, 2, 1, bool(causal), blk, blocks=causal == 2, topk2=1)
                cnt = ctypes.c_int64(0)
                rc = L.muse_plan(N, ctypes.byref(cfg), None, 0, ctypes.byref(cnt))
                if rc == 0 and cnt.value <= 4096:
                    M.plan(N, cfg)
                n += 1
    # layouts: shapes x cluster counts x schemes x dtypes
    for (B, Hq, Hkv, N, D) in ((1, 1, 1, 1, 64), (1, 2, 1, 100, 128), (2, 8, 2, 4096, 64), (1, 32, 8, 65536, 64),
                               (3, 6, 3, 777, 128)):
        for cq, ck in ((1, 1), (16, 16), (24, 80), (256, 3), (256, 256)):
            for topk in (0, 1, 8, 300):
                for causal, blk in ((0, 0), (1, 64), (1, 1000), (2, 64), (2, 1024)):
                    for dt in (0, 1):
                        cfg = M.make_cfg(cq, 3, topk, bool(causal), blk, ck=ck, blocks=causal == 2,
                                         topk2=2, tilt="exact" if causal == 2 else None)
                        lay = M.muse_layout()
                        L.muse_layout_query(B, Hq, Hkv, N, D, dt, ctypes.byref(cfg), ctypes.byref(lay))
                        L.muse_bwd_ws_size(B, Hq, Hkv, N, D, dt, ctypes.byref(cfg))
                        n += 1
    # entry points that fail their checks before queueing anything
    cfg = M.make_cfg(16, 3, 1)
    for args in ((FAKE, FAKE, FAKE, 1, 1, 2, 2, 256, 64, ctypes.byref(cfg), None, None, FAKE, FAKE, FAKE, 16,
                  FAKE, 1 << 40, None),
                 (FAKE, FAKE, FAKE, 1, 1, 2, 2, 256, 96, ctypes.byref(cfg), None, None, FAKE, FAKE, FAKE, 1 << 40,
                  FAKE, 1 << 40, None),
                 (None, FAKE, FAKE, 1, 1, 2, 2, 256, 64, ctypes.byref(cfg), None, None, FAKE, FAKE, FAKE, 1 << 40,
                  FAKE, 1 << 40, None)):
        assert L.museattn_fwd(*args) < 0
    big = M.make_cfg(32, 10, 0, True, 512)
    assert L.museattn_fwd_noalloc(FAKE, FAKE, FAKE, 1, 4, 8, 8, 16384, 64, ctypes.byref(big), None, None, FAKE,
                                  FAKE, FAKE, 1 << 40, None) == -2
    assert L.musecluster(FAKE, 1, 2, 100, 48, 8, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == -1
    assert L.musecluster(FAKE, 1, 2, 100000, 64, 64, 3, None, FAKE, FAKE, FAKE, FAKE, FAKE, 8, None) == -2
    assert L.musesummarize(FAKE, FAKE, 1, 2, 100, 64, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert L.museattn_bwd(None, None, None, None, None, None, 1, 1, 4, 2, 1000, 64, ctypes.byref(cfg), None, 0,
                          None, None, None, None, 0, None) == -1
    for code in (0, -1, -2, -3, -4, 5):
        L.muse_strerror(code)
    L.muse_timing_enable(1); L.muse_timing_collect(); L.muse_timing_reset(); L.muse_timing_enable(0)
    print("host calls under the sanitizer:", n)
""")


def test_host_abi_under_address_sanitizer(tmp_path):
    obj = tmp_path / "capi.o"
    lib = tmp_path / "libmuse_asan.so"
    flags = ["--offload-arch=gfx950", "-O1", "-fPIC", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc")]
    subprocess.run([HIPCC, *flags, *HOST_ASAN, "-c", os.path.join(PKG, "csrc", "capi.hip"), "-o", str(obj)],
                   check=True, capture_output=True)
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *HOST_ASAN, "-o", str(lib), str(obj),
                    *_objects()], check=True, capture_output=True)
    code = f"ROOT = {ROOT!r}\nLIB = {str(lib)!r}\n" + CHILD
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=_env(), timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "AddressSanitizer" not in r.stderr
    assert "host calls under the sanitizer:" in r.stdout
