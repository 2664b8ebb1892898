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
DEBUG_LIB = os.path.join(HERE, "libcakv_debug.so")  # beside libcakv.so: both ship with the tree
PROBES_LIB = os.path.join(HERE, "libcakv_probes.so")  # attainable-peak probes (measurement only)
SOURCES = ["api.hip", "kv_compress.hip", "kv_prepare.hip", "decode.hip", "indexer.hip", "attention.hip", "backward.hip"]
PROBE_SOURCES = ["probes.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# -packed-fp32-ops: hipcc must not emit v_pk_{add,mul,fma}_f32 on its own
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(ROOT, "include")]


def _compile(src: str, objdir: str, extra=()) -> str:
    obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    return obj


def _link(objs, out: str) -> None:
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile every source and link libcakv.so; returns its path.  The
    regular build also links the measurement probes, libcakv_probes.so.
    With debug=True, the debug build instead: the same sources with the
    kernels' device-side index checks compiled in (-DCAKV_DEBUG), as
    libcakv_debug.so (objects in _build/debug/)."""
    objdir = os.path.join(HERE, "_build", "debug") if debug else os.path.join(HERE, "_build")
    out = DEBUG_LIB if debug else LIB
    os.makedirs(objdir, exist_ok=True)
    extra = ["-DCAKV_DEBUG"] if debug else []
    srcs = SOURCES if debug else SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=min(4, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(lambda s: _compile(s, objdir, extra), srcs))
    if not debug:
        _link(objs[len(SOURCES):], PROBES_LIB)
        objs = objs[:len(SOURCES)]
        if verbose:
            print("built", PROBES_LIB)
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


def asan_runtime() -> str:
    """Path of the ROCm clang's shared ASan runtime (to preload into a host
    process that loads a sanitized library)."""
    r = subprocess.run([os.path.join(os.path.dirname(HIPCC), "..", "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isfile(path):
        raise RuntimeError("clang's shared ASan runtime was not found")
    return path


def build_sanitized(out_dir: str) -> str:
    """A copy of libcakv.so whose host code in api.hip (argument validation,
    workspace sizing, launch geometry, the static-scratch lookup) is built
    with AddressSanitizer and UndefinedBehaviorSanitizer; the device code is
    not instrumented (the sanitizer flags reach the host pass only), and the
    other sources' objects come from the regular build.  Returns its path."""
    objdir = os.path.join(HERE, "_build")
    objs = [os.path.join(objdir, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "api.hip"]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise FileNotFoundError("regular build objects missing: " + ", ".join(missing))
    host_san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    api_obj = os.path.join(out_dir, "api_sanitized.o")
    flags = [f if f != "-O3" else "-O1" for f in FLAGS]
    cmd = [HIPCC, *flags, "-g", *host_san, "-c", os.path.join(CSRC, "api.hip"), "-o", api_obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for the sanitized api.hip:\n" + r.stdout + r.stderr)
    lib = os.path.join(out_dir, "libcakv_sanitized.so")
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", api_obj, *objs,
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-shared-libasan", "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed for the sanitized library:\n" + r.stdout + r.stderr)
    return lib


if __name__ == "__main__":
    build(verbose=True, debug="--debug" in sys.argv[1:])
    sys.exit(0)
