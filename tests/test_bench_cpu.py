"""bench.py's host-side contract, on the CPU: it measures one GPU and says so
when asked for more (before it touches a GPU), the source digest that keys
the committed profiles covers exactly libcakv.so's sources and headers (not
the measurement probes), and every committed profile summary was taken at
the current digest, so the line's traffic and rocprof figures resolve."""
import hashlib
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from compressed_attention_kv_amd.build import CSRC, PROBE_SOURCES, SOURCES  # noqa: E402


@pytest.mark.parametrize("args,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_is_refused(args, env):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, capture_output=True,
                       text=True, timeout=300, env=dict(os.environ, **env))
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_source_digest_covers_the_library_sources_only():
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith(".hpp") or f in SOURCES:
            h.update(f.encode())
            h.update(open(os.path.join(CSRC, f), "rb").read())
    assert bench._source_digest() == h.hexdigest()
    assert set(PROBE_SOURCES).isdisjoint(SOURCES)
    assert all(os.path.exists(os.path.join(CSRC, f)) for f in SOURCES + PROBE_SOURCES)


def test_committed_profiles_match_the_current_sources():
    digest = bench._source_digest()
    names = [f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.endswith("_kernels.md")]
    assert len(names) >= 9
    for f in names:
        text = open(os.path.join(ROOT, "profiles", f)).read()
        found = re.findall(r"source_sha256=([0-9a-f]{64})", text)
        assert found and set(found) == {digest}, f
        wl = f[: -len("_kernels.md")]
        kern = re.search(r"duration_us: kernel=(\S+)", text).group(1)
        assert bench._profiled(wl, kern, "duration_us") is not None, f
