"""The C-ABI library loads on a machine without a GPU, exports every function
include/cakv.h declares, and rejects bad arguments on the host before any
HIP call (no compute runs here)."""
import ctypes
import os
import re

import pytest

import compressed_attention_kv_amd as cakv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "cakv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cakv_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return cakv.load_library()


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(cakv.EXPORTS)
    assert cakv.version() == 100


def _prm(**kw):
    d = dict(m=4, n_win=128, rope_dims=64, rope_base=10000.0, softmax_scale=0.0,
             rms_eps=1e-6, gamma_q=None)
    d.update(kw)
    return cakv.AttnParams(**d)


FAKE = 0x10000  # 16-byte aligned non-NULL address; validation rejects before it is touched


def _sparse(lib, prm, **kw):
    a = dict(q=FAKE, kv_c=FAKE, idx=FAKE, kv_raw=FAKE, raw0=FAKE, qpos=FAKE, sinks=FAKE, act=cakv.BF16, B=1,
             Q=1, H=128, D=512, N=16, K=1024, R=4, out=FAKE, odt=cakv.BF16, lse=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.cakv_sparse_mqa_fwd(ctypes.byref(prm), a["q"], a["kv_c"], a["idx"], a["kv_raw"], a["raw0"],
                                   a["qpos"], a["sinks"], a["act"], a["B"], a["Q"], a["H"], a["D"], a["N"], a["K"],
                                   a["R"], a["out"], a["odt"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=96), -2), (dict(H=0), -2), (dict(H=129), -2), (dict(q=None), -1), (dict(q=FAKE + 4), -1),
    (dict(act=cakv.FP8_E4M3), -1), (dict(odt=7), -1), (dict(K=-1), -2), (dict(wsb=0), -3), (dict(ws=None), -3),
    (dict(B=-1), -1),
])
def test_sparse_attention_argument_errors(lib, kw, code):
    assert _sparse(lib, _prm(), **kw) == code
    assert lib.cakv_last_error().decode() != ""


@pytest.mark.parametrize("prm,code", [(_prm(rope_dims=66), -2), (_prm(rope_dims=3), -2), (_prm(m=0), -2),
                                      (_prm(n_win=-1), -2), (_prm(rope_base=0.0), -1), (_prm(rms_eps=-1.0), -1)])
def test_attention_param_errors(lib, prm, code):
    assert _sparse(lib, prm) == code


def test_empty_batch_is_a_no_op(lib):
    assert _sparse(lib, _prm(), B=0, q=None, out=None, ws=None, wsb=0) == 0
    assert lib.cakv_kv_compress(None, cakv.BF16, None, 0, 128, 512, 4, None, cakv.BF16, None, None) == 0


def test_kv_compress_errors(lib):
    f = lib.cakv_kv_compress
    assert f(FAKE, cakv.BF16, FAKE, 1, 8, 512, 0, FAKE, cakv.BF16, None, None) == -2  # m
    assert f(FAKE, cakv.BF16, FAKE, 1, 8, 510, 4, FAKE, cakv.BF16, None, None) == -2  # D % 4
    assert f(FAKE, cakv.BF16, FAKE, 1, 8, 512, 4, FAKE, cakv.FP8_E4M3, None, None) == -1  # scale missing
    assert f(FAKE, cakv.BF16, FAKE, 1, 8, 512, 4, FAKE, cakv.BF16, FAKE, None) == -1  # scale not wanted
    assert f(None, cakv.BF16, FAKE, 1, 8, 512, 4, FAKE, cakv.BF16, None, None) == -1


def test_kv_prepare_errors(lib):
    f = lib.cakv_kv_prepare
    ok = dict(i=FAKE, o=FAKE, dt=cakv.BF16, B=1, N=8, D=512, j0=0, n=8, g=None, m=4, r=64, base=10000.0, off=0,
              eps=1e-6)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["i"], a["o"], a["dt"], a["B"], a["N"], a["D"], a["j0"], a["n"], a["g"], a["m"], a["r"],
                 a["base"], a["off"], a["eps"], None)
    assert call(j0=4, n=5) == -1          # entries past N
    assert call(n=-1) == -1
    assert call(D=500) == -2              # D % 8
    assert call(D=8192) == -2
    assert call(dt=cakv.FP8_E4M3) == -1
    assert call(r=3) == -1 and call(r=520) == -1
    assert call(m=0) == -1
    assert call(base=0.0) == -1 and call(eps=-1.0) == -1
    assert call(i=None) == -1 and call(o=FAKE + 8) == -1 and call(g=FAKE + 4) == -1
    assert call(N=1 << 30, n=1, m=4) == -1  # positions beyond int32
    assert call(B=0, i=None, o=None) == 0 and call(n=0, i=None, o=None) == 0  # nothing to do


def test_indexer_errors_and_workspace(lib):
    f = lib.cakv_indexer_topk
    ws = lib.cakv_indexer_topk_workspace(8, 1, 262144, 1024)
    assert ws >= 8 * 262144 * 4
    assert lib.cakv_indexer_topk_workspace(8, 1, 262144, 2048) >= ws
    # dtype combinations
    assert f(FAKE, cakv.F32, FAKE, FAKE, cakv.FP8_E4M3, FAKE, FAKE, 1, 1, 64, 64, 128, 4, 16, FAKE, FAKE, ws, None) == -2
    assert f(FAKE, cakv.BF16, FAKE, FAKE, cakv.FP8_E4M3, FAKE, FAKE, 1, 1, 64, 48, 128, 4, 16, FAKE, FAKE, ws, None) == -2
    assert f(FAKE, cakv.BF16, FAKE, FAKE, cakv.FP8_E4M3, FAKE, FAKE, 1, 1, 64, 64, 128, 4, 0, FAKE, FAKE, ws, None) == -2
    assert f(FAKE, cakv.BF16, FAKE, FAKE, cakv.FP8_E4M3, FAKE, FAKE, 1, 1, 64, 64, 128, 4, 16, FAKE, FAKE, 0, None) == -3
    assert f(FAKE, cakv.F32, FAKE, FAKE, cakv.F32, FAKE, FAKE, 1, 1, 64, 4, 32, 4, 16, FAKE, FAKE, 1 << 20, None) == -1


def test_workspace_queries_are_monotone(lib):
    a = lib.cakv_sparse_mqa_workspace(32, 1, 128, 512, 1024, 128)
    b = lib.cakv_dense_mqa_workspace(32, 1, 128, 512, 8192, 128)
    assert a > 0 and b > 0
    assert lib.cakv_sparse_mqa_workspace(64, 1, 128, 512, 1024, 128) >= a
    # enough queries to fill the GPU with one split each: no partials, no workspace
    assert lib.cakv_sparse_mqa_workspace(1, 8192, 128, 512, 1024, 128) == 0


def test_profile_kernel_events_arguments(lib):
    # n < 0 and NULL event arrays are rejected on the host; n = 0 clears
    assert lib.cakv_profile_kernel_events(b"mqa_fwd_kernel", None, None, -1) == -1
    assert lib.cakv_profile_kernel_events(b"mqa_fwd_kernel", None, None, 2) == -1
    null2 = (ctypes.c_void_p * 2)(None, None)
    assert lib.cakv_profile_kernel_events(b"mqa_fwd_kernel", null2, null2, 2) == -1
    assert lib.cakv_profile_kernel_events(None, None, None, 0) == 0
