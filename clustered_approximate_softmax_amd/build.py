"""Build the HIP library libmuse.so for gfx950 in-tree (hipcc, no JIT)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "_build")
LIB = os.path.join(OUT, "libmuse.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-fPIC", "-std=c++17",
    # packed fp32 arithmetic off for all device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", SRC,
    "-Wno-unused-result",
]


# per-source extra flags: the attention kernels keep MFMA accumulators in
# VGPRs (no copies between accumulation and arithmetic registers)
EXTRA = {"attn.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return sorted(f for f in os.listdir(SRC) if f.endswith(".hip"))


def _compile(name):
    obj = os.path.join(OUT, name[:-4] + ".o")
    cmd = [HIPCC, *FLAGS, *EXTRA.get(name, []), "-c", os.path.join(SRC, name), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    return name, r.returncode, msg, obj


def build(verbose=True) -> str:
    os.makedirs(OUT, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 4)) as ex:
        res = list(ex.map(_compile, sources()))
    failed = [r for r in res if r[1] != 0]
    for name, rc, msg, _ in res:
        if msg.strip() and (verbose or rc):
            print(f"--- {name}\n{msg}", file=sys.stderr)
    if failed:
        raise RuntimeError("hipcc failed for: " + ", ".join(r[0] for r in failed))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + [r[3] for r in res]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
