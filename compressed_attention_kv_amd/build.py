"""Build the HIP library libcakv.so in-tree for gfx950 (hipcc, no JIT)."""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libcakv.so")
SOURCES = ["api.hip", "kv_compress.hip", "kv_prepare.hip", "indexer.hip", "attention.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: hipcc must not emit v_pk_{add,mul,fma}_f32 on its own
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def _compile(src: str, objdir: str) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libcakv.so; returns its path."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir), SOURCES))
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
