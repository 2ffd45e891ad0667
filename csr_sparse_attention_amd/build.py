"""Builds libcsrsa.so (HIP kernels + C ABI) for gfx950 with hipcc.

    python csr_sparse_attention_amd/build.py

Every source under csrc/ is compiled in parallel into _build/ at the repository
root, then linked into csr_sparse_attention_amd/libcsrsa.so.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(ROOT, "_build", "csrsa")
LIB = os.path.join(PKG, "libcsrsa.so")

ARCH = "gfx950"
HIP_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Wno-unused-lambda-capture",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcsrsa.so)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith((".hip", ".cpp")))


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc()] + HIP_FLAGS + ["-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd = [hipcc(), "-x", "hip"] + HIP_FLAGS + ["-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compiling {os.path.basename(src)} failed:\n{res.stderr}")
    noise = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return obj


def build(jobs: int | None = None) -> str:
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"linking libcsrsa.so failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
