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
    # CAKV_TEST_LIBRARY: run these checks against another build of the same
    # sources (the sanitizer test uses it); the first load is the one cached
    return cakv.load_library(os.environ.get("CAKV_TEST_LIBRARY", cakv.LIB_PATH))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(cakv.EXPORTS)
    assert cakv.version() == 100


def _prm(**kw):
    d = dict(m=4, n_win=128, rope_dims=64, rope_base=10000.0, softmax_scale=0.0,
             rms_eps=1e-6, gamma_q=None, raw_ring=0)
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


def test_indexer_workspace_holds_the_packed_keys(lib):
    """With several queries per sequence the indexer workspace also holds the
    keys repacked for the score kernel, B * ceil(N/32) * 4 KiB (sized for
    128-dim keys), beyond what the same number of one-query sequences
    needs; the size grows with B, Q and N."""
    ws = lib.cakv_indexer_topk_workspace
    for B, Q, N in [(1, 8192, 67584), (2, 3, 5000), (4, 2, 33), (1, 2, 1)]:
        extra = ws(B, Q, N, 1024) - ws(B * Q, 1, N, 1024)
        packed = B * ((N + 31) // 32) * 32 * 128
        assert packed <= extra <= packed + 256, (B, Q, N)
    sizes = [ws(B, Q, N, 1024) for B, Q, N in [(1, 1, 1000), (1, 2, 1000), (1, 3, 1000), (2, 3, 1000), (2, 3, 1001)]]
    assert sizes == sorted(sizes)
    assert ws(3, 1, 0, 64) > 0 and ws(1, 4, 0, 64) == ws(4, 1, 0, 64)  # no keys: nothing to pack


def test_workspace_queries_are_monotone(lib):
    a = lib.cakv_sparse_mqa_workspace(32, 1, 128, 512, 1024, 128)
    b = lib.cakv_dense_mqa_workspace(32, 1, 128, 512, 8192, 128)
    assert a > 0 and b > 0
    assert lib.cakv_sparse_mqa_workspace(64, 1, 128, 512, 1024, 128) >= a
    # a large batch runs one split per query (no partials), but the reported
    # size still covers every smaller batch, so it is not smaller than B*Q=32's
    assert lib.cakv_sparse_mqa_workspace(1, 8192, 128, 512, 1024, 128) >= a


def test_profile_kernel_events_arguments(lib):
    # n < 0 and NULL event arrays are rejected on the host; n = 0 clears
    assert lib.cakv_profile_kernel_events(b"mqa_fwd_kernel", None, None, -1) == -1
    assert lib.cakv_profile_kernel_events(b"mqa_fwd_kernel", None, None, 2) == -1
    null2 = (ctypes.c_void_p * 2)(None, None)
    assert lib.cakv_profile_kernel_events(b"mqa_fwd_kernel", null2, null2, 2) == -1
    assert lib.cakv_profile_kernel_events(None, None, None, 0) == 0


# ---------------------------------------------------------------- documented limits
# Every size include/cakv.h calls supported is accepted and every other one is
# refused.  "Accepted" is checked with an empty batch: sizes are validated
# before the empty-batch return, and nothing is launched.

@pytest.mark.parametrize("act,D,ok", [(cakv.BF16, 128, True), (cakv.BF16, 512, True), (cakv.F32, 128, True),
                                      (cakv.F32, 512, False), (cakv.BF16, 64, False), (cakv.BF16, 256, False),
                                      (cakv.BF16, 96, False), (cakv.BF16, 1024, False), (cakv.F32, 64, False)])
def test_attention_head_dims(lib, act, D, ok):
    rc = _sparse(lib, _prm(), B=0, act=act, D=D)
    assert rc == (0 if ok else -2)
    rc = lib.cakv_dense_compressed_mqa_fwd(ctypes.byref(_prm()), None, None, None, None, None, None, act, 0, 1, 128,
                                           D, 16, 4, None, cakv.BF16, None, None, 0, None)
    assert rc == (0 if ok else -2)


@pytest.mark.parametrize("H,ok", [(1, True), (5, True), (64, True), (128, True), (0, False), (129, False)])
def test_attention_head_counts(lib, H, ok):
    assert _sparse(lib, _prm(), B=0, H=H) == (0 if ok else -2)


@pytest.mark.parametrize("K,ok", [(0, True), (1, True), (65536, True), (-1, False), (65537, False)])
def test_attention_topk_slots(lib, K, ok):
    assert _sparse(lib, _prm(), B=0, K=K) == (0 if ok else -2)


@pytest.mark.parametrize("kw,ok", [(dict(m=1), True), (dict(m=4096), True), (dict(m=4097), False),
                                   (dict(n_win=0), True), (dict(n_win=4096), True), (dict(n_win=4097), False),
                                   (dict(rope_dims=0), True), (dict(rope_dims=64), True),
                                   (dict(rope_dims=66), False), (dict(rope_dims=7), False)])
def test_attention_param_limits(lib, kw, ok):
    assert _sparse(lib, _prm(**kw), B=0) == (0 if ok else -2)


def _indexer(lib, qdt, kdt, HI, dI, k, ks=None, B=0):
    return lib.cakv_indexer_topk(None, qdt, None, None, kdt, ks, None, B, 1, 64, HI, dI, 4, k, None, None, 0, None)


@pytest.mark.parametrize("HI,dI,ok", [(32, 64, True), (32, 128, True), (64, 64, True), (64, 128, True),
                                      (16, 128, False), (48, 128, False), (128, 128, False), (64, 32, False),
                                      (64, 96, False), (64, 256, False)])
def test_indexer_bf16_mode_sizes(lib, HI, dI, ok):
    assert _indexer(lib, cakv.BF16, cakv.FP8_E4M3, HI, dI, 1024) == (0 if ok else -2)


@pytest.mark.parametrize("HI,dI,ok", [(1, 4, True), (4, 32, True), (64, 128, True), (8, 1024, True),
                                      (64, 129, False), (65, 32, False), (0, 32, False), (64, 132, False),
                                      (4, 2, False)])
def test_indexer_fp32_mode_sizes(lib, HI, dI, ok):
    assert _indexer(lib, cakv.F32, cakv.F32, HI, dI, 64) == (0 if ok else -2)


@pytest.mark.parametrize("k,ok", [(1, True), (1024, True), (4096, True), (0, False), (4097, False)])
def test_indexer_k_range(lib, k, ok):
    assert _indexer(lib, cakv.BF16, cakv.FP8_E4M3, 64, 128, k) == (0 if ok else -2)


@pytest.mark.parametrize("qdt,kdt", [(cakv.F32, cakv.FP8_E4M3), (cakv.BF16, cakv.F32), (cakv.BF16, cakv.BF16)])
def test_indexer_mode_dtypes(lib, qdt, kdt):
    assert _indexer(lib, qdt, kdt, 64, 128, 64) == -2


@pytest.mark.parametrize("xdt", [cakv.F32, cakv.BF16])
@pytest.mark.parametrize("D,ok", [(4, True), (8, True), (12, True), (512, True), (4096, True), (2, False),
                                  (510, False), (4100, False)])
def test_kv_compress_dims(lib, xdt, D, ok):
    rc = lib.cakv_kv_compress(None, xdt, None, 0, 8, D, 4, None, cakv.BF16, None, None)
    assert rc == (0 if ok else -2)


@pytest.mark.parametrize("m,ok", [(1, True), (4, True), (128, True), (4096, True), (0, False), (4097, False)])
def test_kv_compress_ratios(lib, m, ok):
    assert lib.cakv_kv_compress(None, cakv.BF16, None, 0, 8, 512, m, None, cakv.BF16, None, None) == (0 if ok else -2)


@pytest.mark.parametrize("D,ok", [(8, True), (64, True), (512, True), (4096, True), (4, False), (12, False),
                                  (4104, False)])
def test_kv_prepare_dims(lib, D, ok):
    rc = lib.cakv_kv_prepare(None, None, cakv.BF16, 0, 8, D, 0, 8, None, 4, 0, 10000.0, 0, 1e-6, None)
    assert rc == (0 if ok else -2)


def test_attention_workspace_never_shrinks_with_the_batch(lib):
    """A workspace sized for the largest batch serves every smaller one: the
    reported size is non-decreasing in B*Q (the split count grows as the batch
    shrinks, so the launch workspace alone is not)."""
    for K, nw in ((1024, 128), (64, 16), (0, 128)):
        sizes = [lib.cakv_sparse_mqa_workspace(1, bq, 128, 512, K, nw) for bq in range(1, 600)]
        assert all(b >= a for a, b in zip(sizes, sizes[1:])), K
    sizes = [lib.cakv_dense_mqa_workspace(bq, 1, 128, 512, 8192, 128) for bq in range(1, 600)]
    assert all(b >= a for a, b in zip(sizes, sizes[1:]))
    assert sizes[-1] > 0


def test_binding_rejects_wrong_element_types():
    """The binding checks element types before calling the library (an int64
    position tensor would otherwise be read as pairs of int32 words)."""
    import torch

    class FakeDev:  # stands in for a device tensor: only the fields _dev reads
        is_cuda = True

        def __init__(self, dtype):
            self.dtype = dtype

        def is_contiguous(self):
            return True

        def data_ptr(self):
            return FAKE

    assert cakv._dev(FakeDev(torch.int32), "q_pos", torch.int32) == FAKE
    with pytest.raises(cakv.CakvError, match="q_pos must be torch.int32"):
        cakv._dev(FakeDev(torch.int64), "q_pos", torch.int32)
    with pytest.raises(cakv.CakvError, match="sinks must be torch.float32"):
        cakv._dev(FakeDev(torch.bfloat16), "sinks", torch.float32)


# ---------------------------------------------------------------- compressor variants and the streaming append

@pytest.mark.parametrize("m,span,pc,ok", [(4, 4, 0, True), (4, 8, 1, True), (128, 8192, 0, True), (4, 3, 0, False),
                                          (4, 8193, 0, False), (0, 4, 0, False)])
def test_kv_compress_ex_spans(lib, m, span, pc, ok):
    rc = lib.cakv_kv_compress_ex(None, cakv.BF16, None, pc, 0, 8, 512, m, span, None, cakv.BF16, None, None)
    assert rc == (0 if ok else -2)


def test_kv_compress_ex_errors(lib):
    f = lib.cakv_kv_compress_ex
    assert f(FAKE, cakv.BF16, FAKE, 2, 1, 8, 512, 4, 4, FAKE, cakv.BF16, None, None) == -1  # gate kind
    assert f(FAKE, cakv.BF16, FAKE, 1, 1, 8, 512, 4, 8, FAKE, cakv.FP8_E4M3, None, None) == -1  # scale missing
    assert f(FAKE, cakv.BF16, None, 1, 1, 8, 512, 4, 8, FAKE, cakv.BF16, None, None) == -1  # gate NULL


def _append(lib, **kw):
    a = dict(x=FAKE, g=FAKE, pc=0, pos=FAKE, act=cakv.BF16, B=2, D=512, raw=FAKE, graw=FAKE, Rr=128, win=FAKE,
             Rw=128, cache=FAKE, cdt=cakv.BF16, cs=None, N=64, m=4, span=4,
             prep=ctypes.byref(cakv.PrepParams(64, 10000.0, 0, 1e-6, None)))
    a.update(kw)
    return lib.cakv_kv_append(a["x"], a["g"], a["pc"], a["pos"], a["act"], a["B"], a["D"], a["raw"], a["graw"],
                              a["Rr"], a["win"], a["Rw"], a["cache"], a["cdt"], a["cs"], a["N"], a["m"], a["span"],
                              a["prep"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0, x=None, pos=None), 0),                                   # nothing to do
    (dict(Rr=3), -1), (dict(span=8, Rr=7), -1),                         # ring shorter than the span
    (dict(cdt=cakv.FP8_E4M3), -1),                                      # fp8 cache: scale required
    (dict(cdt=cakv.FP8_E4M3, cs=FAKE), -1),                             # ... and no preparation
    (dict(cdt=cakv.FP8_E4M3, cs=FAKE, prep=None, win=None, B=0, x=None), 0),
    (dict(cdt=cakv.F32), -1),                                           # cache type differs from the tokens'
    (dict(prep=None), -1),                                              # a window ring needs preparation
    (dict(D=500), -2), (dict(D=8192), -2), (dict(m=0), -2), (dict(span=3), -2),
    (dict(pc=2), -1), (dict(x=None), -1), (dict(raw=FAKE + 4), -1),
    (dict(prep=ctypes.byref(cakv.PrepParams(63, 10000.0, 0, 1e-6, None))), -1),
    (dict(N=1 << 30, m=4), -1),                                          # entry positions beyond int32
])
def test_kv_append_errors(lib, kw, code):
    assert _append(lib, **kw) == code


def test_attention_ring_mode_needs_a_window_sized_ring(lib):
    assert _sparse(lib, _prm(raw_ring=1), B=0, R=64) == -1      # n_win = 128 > R
    assert _sparse(lib, _prm(raw_ring=1), B=0, R=128) == 0
    assert _sparse(lib, _prm(raw_ring=1), raw0=None, R=128, B=0) == 0
    assert _sparse(lib, _prm(raw_ring=2), B=0, R=128) == -1


# ---------------------------------------------------------------- backward entry points

def _mqa_bwd(lib, **kw):
    a = dict(q=FAKE, kv_c=FAKE, idx=FAKE, kv_raw=FAKE, raw0=FAKE, qpos=FAKE, sinks=FAKE, act=cakv.BF16, B=1, Q=1,
             H=128, D=512, N=16, K=64, R=128, out=FAKE, odt=cakv.F32, lse=FAKE, dout=FAKE, dq=FAKE, dkc=FAKE,
             dkr=FAKE, ds=None, dg=None, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.cakv_mqa_bwd(ctypes.byref(_prm()), a["q"], a["kv_c"], a["idx"], a["kv_raw"], a["raw0"], a["qpos"],
                            a["sinks"], a["act"], a["B"], a["Q"], a["H"], a["D"], a["N"], a["K"], a["R"], a["out"],
                            a["odt"], a["lse"], a["dout"], a["dq"], a["dkc"], a["dkr"], a["ds"], a["dg"], a["ws"],
                            a["wsb"], None)


@pytest.mark.parametrize("kw,code", [(dict(B=0, q=None), 0), (dict(D=128), -2), (dict(act=cakv.F32, D=128), -2),
                                     (dict(H=129), -2), (dict(lse=None), -1), (dict(dout=None), -1),
                                     (dict(dq=None), -1), (dict(dkc=None), -1), (dict(dkr=None), -1),
                                     (dict(wsb=0), -3), (dict(ws=None), -3), (dict(K=65537), -2),
                                     (dict(B=70000), -2), (dict(ds=FAKE + 4), -1)])
def test_mqa_bwd_argument_errors(lib, kw, code):
    assert _mqa_bwd(lib, **kw) == code


def test_mqa_bwd_workspace_never_shrinks_with_the_batch(lib):
    sizes = [lib.cakv_mqa_bwd_workspace(1, bq, 128, 512, 1024, 128) for bq in range(1, 400)]
    assert all(b >= a for a, b in zip(sizes, sizes[1:])) and sizes[0] > 0


def test_kv_prepare_bwd_and_compress_bwd_errors(lib):
    f = lib.cakv_kv_prepare_bwd
    assert f(FAKE, cakv.BF16, FAKE, FAKE, None, 1, 8, 500, 0, 8, None, 4, 64, 10000.0, 0, 1e-6, None) == -2
    assert f(FAKE, cakv.BF16, None, FAKE, None, 1, 8, 512, 0, 8, None, 4, 64, 10000.0, 0, 1e-6, None) == -1
    assert f(FAKE, cakv.BF16, FAKE, FAKE, None, 1, 8, 512, 4, 8, None, 4, 64, 10000.0, 0, 1e-6, None) == -1
    assert f(None, cakv.BF16, None, None, None, 0, 8, 512, 0, 8, None, 4, 64, 10000.0, 0, 1e-6, None) == 0
    g = lib.cakv_kv_compress_bwd
    ws = lib.cakv_kv_compress_bwd_workspace(1, 64, 512, 4)
    assert ws == 16 * 512 * 12
    assert g(FAKE, cakv.BF16, FAKE, 0, 1, 64, 512, 4, 3, FAKE, FAKE, FAKE, FAKE, ws, None) == -2  # span < m
    assert g(FAKE, cakv.BF16, FAKE, 0, 1, 64, 512, 4, 4, FAKE, FAKE, FAKE, FAKE, 0, None) == -3
    assert g(FAKE, cakv.BF16, FAKE, 0, 1, 64, 512, 4, 4, None, FAKE, FAKE, FAKE, ws, None) == -1
    assert g(None, cakv.BF16, None, 0, 0, 64, 512, 4, 4, None, None, None, None, 0, None) == 0


@pytest.mark.parametrize("kw,code", [(dict(), 0), (dict(HI=65), -2), (dict(dI=136), -2), (dict(dI=132), -2),
                                     (dict(dI=64), 0), (dict(dI=20), -2),
                                     (dict(qdt=cakv.F32), -2), (dict(ks=None), -1), (dict(K=65537), -2)])
def test_indexer_bwd_limits(lib, kw, code):
    a = dict(qdt=cakv.BF16, kdt=cakv.FP8_E4M3, ks=FAKE, HI=64, dI=128, K=1024)
    a.update(kw)
    # an empty batch validates the sizes and launches nothing
    rc = lib.cakv_indexer_bwd(None, a["qdt"], None, None, a["kdt"], a["ks"], None, None, None, 0, 1, 64, a["HI"],
                              a["dI"], 4, a["K"], None, None, None, None)
    assert rc == code


def test_indexer_bwd_batch_limit(lib):
    # one workgroup column per query: B*Q must stay below 2^23 (checked before any pointer)
    rc = lib.cakv_indexer_bwd(None, cakv.BF16, None, None, cakv.FP8_E4M3, FAKE, None, None, None, 1 << 23, 1, 64, 64,
                              128, 4, 1024, None, None, None, None)
    assert rc == -2
    rc = lib.cakv_indexer_bwd(None, cakv.BF16, None, None, cakv.FP8_E4M3, FAKE, None, None, None, (1 << 23) - 1, 1,
                              64, 64, 128, 4, 1024, None, None, None, None)
    assert rc == -1  # within the limit: the NULL q_idx is the first error


# ------------------------------------------------------------------ measurement probes

def _probe_functions():
    src = open(os.path.join(ROOT, "include", "cakv_probes.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(cakv_[a-z0-9_]+)\s*\(", src)))


def test_probes_library_exports_its_declared_symbols():
    p = cakv.load_probes()
    names = _probe_functions()
    assert set(names) == set(cakv.PROBE_EXPORTS) and len(names) == 2
    for n in names:
        assert hasattr(p, n), n


@pytest.mark.parametrize("buf,nbytes,sink,blocks", [
    (None, 16, FAKE, 1), (FAKE, 16, None, 1), (FAKE + 4, 16, FAKE, 1), (FAKE, 24, FAKE, 1),
    (FAKE, 16, FAKE, -1), (FAKE, 16, FAKE, 65536)])
def test_probe_read_rejects_bad_arguments(buf, nbytes, sink, blocks):
    assert cakv.load_probes().cakv_probe_read(buf, nbytes, sink, blocks, None) == -1


@pytest.mark.parametrize("iters,blocks,sink", [(-1, 1, FAKE), (1, 0, FAKE), (1, 65536, FAKE), (1, 1, None)])
def test_probe_mfma_rejects_bad_arguments(iters, blocks, sink):
    assert cakv.load_probes().cakv_probe_mfma_bf16(iters, blocks, sink, None) == -1


# ------------------------------------------------------------------ batched appends

def test_append_call_layout(tmp_path):
    """The binding's mirror of cakv_append_call has the C compiler's layout
    (size and every field's offset, from a program built against cakv.h)."""
    import subprocess
    fields = [f for f, _ in cakv.AppendCall._fields_]
    src = tmp_path / "layout.c"
    src.write_text("#include <stdio.h>\n#include <stddef.h>\n#include \"cakv.h\"\nint main(void) {\n"
                   "  printf(\"%zu\\n\", sizeof(cakv_append_call));\n" +
                   "".join(f"  printf(\"%zu\\n\", offsetof(cakv_append_call, {f}));\n" for f in fields) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(cakv.AppendCall)
    assert got[1:] == [getattr(cakv.AppendCall, f).offset for f in fields]


def _append_call(**kw):
    d = dict(x_tok=FAKE, gate_tok=FAKE, gate_per_channel=0, act_dtype=cakv.BF16, D=512, raw_ring=FAKE,
             gate_ring=FAKE + 0x100, Rr=8, win_ring=None, Rw=0, cache=FAKE + 0x200, cache_dtype=cakv.BF16, m=4,
             cache_scale=None, N=16, span=4, prep=None)
    d.update(kw)
    return cakv.AppendCall(**d)


@pytest.mark.parametrize("calls,n,code", [
    (None, 1, -1),
    ([_append_call()], 0, -1),
    ([_append_call()] * 5, 5, -1),
    ([_append_call(D=7)], 1, -2),
    ([_append_call(cache_dtype=cakv.FP8_E4M3)], 1, -1),  # fp8 without its scale
    ([_append_call(), _append_call()], 2, -1),           # two appends writing the same rings
    ([_append_call(), _append_call(raw_ring=FAKE + 0x300, gate_ring=FAKE + 0x400)], 2, -1),  # the same cache
])
def test_append_batch_rejects_bad_arguments(lib, calls, n, code):
    arr = None if calls is None else (cakv.AppendCall * len(calls))(*calls)
    assert lib.cakv_kv_append_batch(arr, n, FAKE, 4, None) == code
    assert lib.cakv_last_error()


def test_append_batch_with_no_tokens_runs_nothing(lib):
    # as cakv_kv_append: B = 0 validates the sizes and launches nothing, NULL buffers included
    calls = (cakv.AppendCall * 2)(_append_call(x_tok=None, gate_tok=None, raw_ring=None, gate_ring=None, cache=None),
                                  _append_call(x_tok=None, gate_tok=None, raw_ring=None, gate_ring=None, cache=None))
    assert lib.cakv_kv_append_batch(calls, 2, None, 0, None) == 0
    assert lib.cakv_kv_append_batch(calls, 2, None, -1, None) == -1
