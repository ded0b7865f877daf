"""Build libattn_mi355x.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: python -m mha_mla_kv_amd.build   (or mha_mla_kv_amd.build.build_library())
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libattn_mi355x.so")
ARCH = "gfx950"

SOURCES = ["attn_api.cpp", "decode_gqa.hip", "decode_mla.hip", "prefill_gqa.hip", "cache_append.hip",
           "rope_append.hip"]

# -packed-fp32-ops off: keep fp32 arithmetic on plain (non-packed) VALU instructions.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(src: str, extra: list[str], build_dir: str) -> str:
    os.makedirs(build_dir, exist_ok=True)
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj] + COMMON + DEVICE_FLAGS + extra
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{out}")
    if out.strip():
        print(out, file=sys.stderr)
    return obj


def build_library(extra: list[str] | None = None, jobs: int = 4, out: str = LIB,
                  build_dir: str = BUILD) -> str:
    """Compile every HIP/C++ source for gfx950 and link the shared library at `out`. Always rebuilds."""
    extra = list(extra or [])
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, build_dir), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library())
