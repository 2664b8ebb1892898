"""CPU oracle of the compressed-attention hot path -- TEST INFRASTRUCTURE.

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg
of ``bench.py`` may import this package.  The product path (the HIP library
and its Python binding) never calls it, and the two share no code.

The arithmetic lives in ``cakv_oracle.c`` (plain C, fp64 except for the
canonical fp32 indexer score); this module only marshals numpy/torch arrays
through ctypes.  See the C file's header for the pages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cakv_oracle.c")
_SO = os.path.join(_HERE, "libcakv_oracle.so")

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-mfma", "-fopenmp", "-shared", "-fPIC", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no contraction)."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + f".tmp{os.getpid()}"
        subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _SO)
    return _SO


def build_sanitized(out_dir: str) -> str:
    """A copy of the oracle built with AddressSanitizer and
    UndefinedBehaviorSanitizer (same arithmetic flags); returns its path.  A
    process loads it with CAKV_ORACLE_LIBRARY set to that path and gcc's
    libasan preloaded."""
    so = os.path.join(out_dir, "libcakv_oracle_sanitized.so")
    flags = [f for f in GCC_FLAGS if f != "-O2"] + ["-O1", "-g", "-fno-omit-frame-pointer",
                                                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    subprocess.run(["gcc", *flags, _SRC, "-o", so, "-lm"], check=True)
    return so


_lib = None
_i64 = ctypes.c_int64
_p = ctypes.c_void_p


class AttnParams(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("n_win", ctypes.c_int32), ("rope_dims", ctypes.c_int32),
                ("entry_pos_offset", ctypes.c_int32), ("rope_base", ctypes.c_double),
                ("softmax_scale", ctypes.c_double), ("rms_eps", ctypes.c_double)]


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("CAKV_ORACLE_LIBRARY")  # another build of the same source (sanitizer runs)
        if not path:
            build(force=False)
            path = _SO
        lib = ctypes.CDLL(path)
        lib.oracle_kv_compress.argtypes = [_p, ctypes.c_int, _p, _i64, _i64, _i64, ctypes.c_int, _p]
        lib.oracle_kv_compress_ex.argtypes = [_p, ctypes.c_int, _p, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int,
                                              ctypes.c_int, _p]
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_int]
        lib.oracle_e4m3_decode.restype = ctypes.c_double
        lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        lib.oracle_q8_quantize.argtypes = [_p, ctypes.c_int, _i64, _i64, _p, _p]
        lib.oracle_indexer_scores.argtypes = [_p, ctypes.c_int, _p, _p, _p, _p, _p, _i64, _i64, _i64,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int, _p, _i64, _p, _p]
        lib.oracle_topk.argtypes = [_p, _p, _i64, _i64, ctypes.c_int, _p]
        lib.oracle_kv_prepare.argtypes = [_p, ctypes.c_int, _p, _i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_double, _p]
        lib.oracle_attention.argtypes = [ctypes.POINTER(AttnParams), _p, _p, _p, ctypes.c_int, _p, _p,
                                         _p, _p, _p, _p, ctypes.c_int, _i64, _i64, _i64, _i64, _i64,
                                         _i64, _p, _i64, _p, _p]
        lib.oracle_kv_prepare_bwd.argtypes = [_p, ctypes.c_int, _p, _i64, _i64, _i64, _i64, _i64, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_double, ctypes.c_int, ctypes.c_double, _p, _p,
                                              _p]
        lib.oracle_kv_compress_bwd.argtypes = [_p, ctypes.c_int, _p, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int,
                                               ctypes.c_int, _p, _p, _p]
        lib.oracle_indexer_bwd.argtypes = [_p, ctypes.c_int, _p, _p, _p, _p, _p, _p, _i64, _i64, _i64, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int, _p, ctypes.c_int, _p, _p, _p]
        lib.oracle_attention_bwd.argtypes = [ctypes.POINTER(AttnParams), _p, _p, _p, ctypes.c_int, _p, _p, _p, _p,
                                             _p, _p, ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _i64, _p, _p, _p,
                                             _p, _p, _p]
        _lib = lib
    return _lib


def _act(t) -> tuple[np.ndarray, int]:
    """(contiguous host array, dtype code): float32 -> 0, bfloat16 bits -> 1."""
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().contiguous()
        if t.dtype == torch.bfloat16:
            return t.view(torch.int16).numpy(), 1
        return t.to(torch.float32).numpy(), 0
    return np.ascontiguousarray(t, dtype=np.float32), 0


def _np(t, dtype) -> np.ndarray:
    if isinstance(t, torch.Tensor):
        t = t.detach().cpu().contiguous().numpy()
    return np.ascontiguousarray(t, dtype=dtype)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid input (rc={rc})")


def kv_compress(x, gate, m: int) -> np.ndarray:
    """Softmax-weighted compression of every m tokens; fp64 [B, T//m, D]."""
    lib = _load()
    xa, xd = _act(x)
    g = _np(gate, np.float32)
    B, T, D = xa.shape
    out = np.empty((B, T // m, D), dtype=np.float64)
    _check(lib.oracle_kv_compress(_ptr(xa), xd, _ptr(g), B, T, D, m, _ptr(out)), "kv_compress")
    return out


def kv_compress_ex(x, gate, m: int, span: int = None) -> np.ndarray:
    """Compression variants: entry j is the softmax-gated sum of the `span`
    tokens ending where block j ends (span >= m, cut at token 0); `gate` is
    [B,T] (one logit per token) or [B,T,D] (one per token and channel).
    fp64 [B, T//m, D]."""
    lib = _load()
    xa, xd = _act(x)
    g = _np(gate, np.float32)
    B, T, D = xa.shape
    per_channel = g.ndim == 3
    if g.shape != ((B, T, D) if per_channel else (B, T)):
        raise ValueError("gate must be [B,T] or [B,T,D]")
    span = m if span is None else span
    out = np.empty((B, T // m, D), dtype=np.float64)
    _check(lib.oracle_kv_compress_ex(_ptr(xa), xd, _ptr(g), int(per_channel), B, T, D, m, span, _ptr(out)),
           "kv_compress_ex")
    return out


def e4m3_decode(code: int) -> float:
    return _load().oracle_e4m3_decode(int(code))


def e4m3_encode(v: float) -> int:
    return _load().oracle_e4m3_encode(float(v))


def q8_quantize(c) -> tuple[np.ndarray, np.ndarray]:
    """Per-row power-of-two scale + E4M3 codes: (codes uint8 [..., D], scale f32 [...])."""
    lib = _load()
    if isinstance(c, torch.Tensor):
        c = c.detach().cpu().numpy()
    is64 = c.dtype == np.float64
    a = np.ascontiguousarray(c, dtype=np.float64 if is64 else np.float32)
    D = a.shape[-1]
    n = a.size // D
    codes = np.empty(a.shape, dtype=np.uint8)
    scale = np.empty(a.shape[:-1], dtype=np.float32)
    _check(lib.oracle_q8_quantize(_ptr(a), int(is64), n, D, _ptr(codes), _ptr(scale)), "q8")
    return codes, scale


def q8_dequantize(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """code * scale as float32 (exact)."""
    table = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float32)
    return table[codes] * scale[..., None]


def _rows(rows, B, Q):
    if rows is None:
        return None, B * Q
    r = np.ascontiguousarray(rows, dtype=np.int64)
    return r, r.size


def indexer_scores(q_idx, w, q_pos, m: int, k_f32=None, k_code=None, k_scale=None, rows=None):
    """Canonical fp32 scores [n_rows, N] (NaN where not visible) and n_vis [n_rows]."""
    lib = _load()
    qa, qd = _act(q_idx)
    B, Q, HI, dI = qa.shape
    wa = _np(w, np.float32)
    qp = _np(q_pos, np.int32)
    if k_code is not None:
        kc = _np(k_code, np.uint8)
        ks = _np(k_scale, np.float32)
        kf = None
        N = kc.shape[1]
    else:
        kf = _np(k_f32, np.float32)
        kc = ks = None
        N = kf.shape[1]
    r, n = _rows(rows, B, Q)
    scores = np.empty((n, N), dtype=np.float32)
    nvis = np.empty((n,), dtype=np.int32)
    _check(lib.oracle_indexer_scores(_ptr(qa), qd, _ptr(wa), _ptr(kf), _ptr(kc), _ptr(ks), _ptr(qp),
                                     B, Q, N, HI, dI, m, _ptr(r), n, _ptr(scores), _ptr(nvis)),
           "indexer_scores")
    return scores, nvis


def topk(scores: np.ndarray, n_vis: np.ndarray, k: int) -> np.ndarray:
    lib = _load()
    s = np.ascontiguousarray(scores, dtype=np.float32)
    nv = np.ascontiguousarray(n_vis, dtype=np.int32)
    n, N = s.shape
    idx = np.empty((n, k), dtype=np.int32)
    _check(lib.oracle_topk(_ptr(s), _ptr(nv), n, N, k, _ptr(idx)), "topk")
    return idx


def indexer_topk(q_idx, w, q_pos, m: int, k: int, k_f32=None, k_code=None, k_scale=None, rows=None):
    s, nv = indexer_scores(q_idx, w, q_pos, m, k_f32=k_f32, k_code=k_code, k_scale=k_scale, rows=rows)
    return topk(s, nv, k)


def kv_prepare(kv_c, *, m: int, rope_dims: int, rope_base: float = 10000.0, entry_pos_offset: int = 0,
               rms_eps: float = 1e-6, gamma_kv=None, j0: int = 0, n=None) -> np.ndarray:
    """Key/value vectors of compressed entries j0 .. j0+n-1 (all by default):
    RMSNorm with gamma_kv, the last rope_dims dims rotated by j*m + entry_pos_offset.
    fp64 [B, n, D]."""
    lib = _load()
    ka, kd = _act(kv_c)
    B, N, D = ka.shape
    n = N - j0 if n is None else n
    gk = None if gamma_kv is None else _np(gamma_kv, np.float32)
    out = np.empty((B, n, D), dtype=np.float64)
    _check(lib.oracle_kv_prepare(_ptr(ka), kd, _ptr(gk), B, N, D, j0, n, m, rope_dims, rope_base,
                                 entry_pos_offset, rms_eps, _ptr(out)), "kv_prepare")
    return out


def attention(q, kv_c, kv_raw, raw_pos0, q_pos, sinks, *, idx=None, m: int, n_win: int,
              rope_dims: int, rope_base: float = 10000.0, entry_pos_offset: int = 0,
              softmax_scale: float = 0.0, rms_eps: float = 1e-6, gamma_q=None, gamma_kv=None,
              rows=None):
    """Sink-augmented MQA over compressed entries (idx given: sparse, else all visible)
    plus the raw window.  Returns (out fp64 [n_rows,H,D], lse fp64 [n_rows,H])."""
    lib = _load()
    qa, qd = _act(q)
    ka, kd = _act(kv_c)
    ra, rd = _act(kv_raw)
    if not (qd == kd == rd):
        raise ValueError("q, kv_c and kv_raw must share one storage type")
    B, Q, H, D = qa.shape
    N = ka.shape[1]
    R = ra.shape[1]
    ia = None
    K = 0
    if idx is not None:
        ia = _np(idx, np.int32)
        K = ia.shape[-1]
    rp = _np(raw_pos0, np.int32)
    qp = _np(q_pos, np.int32)
    sk = _np(sinks, np.float32)
    gq = None if gamma_q is None else _np(gamma_q, np.float32)
    gk = None if gamma_kv is None else _np(gamma_kv, np.float32)
    r, n = _rows(rows, B, Q)
    out = np.empty((n, H, D), dtype=np.float64)
    lse = np.empty((n, H), dtype=np.float64)
    prm = AttnParams(m, n_win, rope_dims, entry_pos_offset, rope_base, softmax_scale, rms_eps)
    _check(lib.oracle_attention(ctypes.byref(prm), _ptr(qa), _ptr(ka), _ptr(ia), K, _ptr(ra), _ptr(rp),
                                _ptr(qp), _ptr(sk), _ptr(gq), _ptr(gk), qd, B, Q, H, D, N, R, _ptr(r), n,
                                _ptr(out), _ptr(lse)), "attention")
    return out, lse


# ---------------------------------------------------------------- backward (training)

def kv_prepare_bwd(kv_c, dy, *, m: int, rope_dims: int, rope_base: float = 10000.0, entry_pos_offset: int = 0,
                   rms_eps: float = 1e-6, gamma_kv=None, j0: int = 0, n=None):
    """Gradient of kv_prepare: dy [B,n,D] of the prepared rows of entries
    j0 .. j0+n-1 -> (dx [B,n,D] of the raw entries, dgamma_kv [D]), fp64."""
    lib = _load()
    ka, kd = _act(kv_c)
    B, N, D = ka.shape
    n = N - j0 if n is None else n
    dya = np.ascontiguousarray(dy, dtype=np.float64)
    assert dya.shape == (B, n, D)
    gk = None if gamma_kv is None else _np(gamma_kv, np.float32)
    dx = np.empty((B, n, D), dtype=np.float64)
    dg = np.empty((D,), dtype=np.float64)
    _check(lib.oracle_kv_prepare_bwd(_ptr(ka), kd, _ptr(gk), B, N, D, j0, n, m, rope_dims, rope_base,
                                     entry_pos_offset, rms_eps, _ptr(dya), _ptr(dx), _ptr(dg)), "kv_prepare_bwd")
    return dx, dg


def kv_compress_bwd(x, gate, m: int, dc, span: int = None):
    """Gradient of kv_compress_ex: dc [B,T//m,D] -> (dx [B,T,D], dgate of the
    gate's shape), fp64."""
    lib = _load()
    xa, xd = _act(x)
    g = _np(gate, np.float32)
    B, T, D = xa.shape
    per_channel = g.ndim == 3
    span = m if span is None else span
    dca = np.ascontiguousarray(dc, dtype=np.float64)
    assert dca.shape == (B, T // m, D)
    dx = np.empty((B, T, D), dtype=np.float64)
    dg = np.empty(g.shape, dtype=np.float64)
    _check(lib.oracle_kv_compress_bwd(_ptr(xa), xd, _ptr(g), int(per_channel), B, T, D, m, span, _ptr(dca),
                                      _ptr(dx), _ptr(dg)), "kv_compress_bwd")
    return dx, dg


def indexer_bwd(q_idx, w, q_pos, m: int, idx, dS, k_f32=None, k_code=None, k_scale=None, absolute=False):
    """Gradient of the indexer score over the selected entries idx [B,Q,K]
    given dS [B,Q,K] -> (dq_idx [B,Q,HI,dI], dw [B,Q,HI], dk [B,N,dI]), fp64;
    ReLU decisions on the canonical fp32 score.  absolute=True sums |terms|."""
    lib = _load()
    qa, qd = _act(q_idx)
    B, Q, HI, dI = qa.shape
    wa = _np(w, np.float32)
    qp = _np(q_pos, np.int32)
    ia = _np(idx, np.int32)
    K = ia.shape[-1]
    dsa = _np(dS, np.float32)
    if k_code is not None:
        kc, ks, kf = _np(k_code, np.uint8), _np(k_scale, np.float32), None
        N = kc.shape[1]
    else:
        kf, kc, ks = _np(k_f32, np.float32), None, None
        N = kf.shape[1]
    dq = np.empty((B, Q, HI, dI), dtype=np.float64)
    dw = np.empty((B, Q, HI), dtype=np.float64)
    dk = np.empty((B, N, dI), dtype=np.float64)
    _check(lib.oracle_indexer_bwd(_ptr(qa), qd, _ptr(wa), _ptr(kf), _ptr(kc), _ptr(ks), _ptr(qp), _ptr(ia), B, Q, N,
                                  HI, dI, m, K, _ptr(dsa), int(absolute), _ptr(dq), _ptr(dw), _ptr(dk)),
           "indexer_bwd")
    return dq, dw, dk


def attention_bwd(q, kv_c, kv_raw, raw_pos0, q_pos, sinks, dout, *, idx=None, m: int, n_win: int, rope_dims: int,
                  rope_base: float = 10000.0, entry_pos_offset: int = 0, softmax_scale: float = 0.0,
                  rms_eps: float = 1e-6, gamma_q=None, gamma_kv=None):
    """Gradient of attention() given dout [B,Q,H,D] (kv_c and kv_raw raw rows,
    prepared inside as the forward does).  Returns a dict of fp64 arrays:
    dq [B,Q,H,D] (raw query heads), dkhat_c [B,N,D] and dkhat_raw [B,R,D]
    (the prepared rows the attention calls read), dsinks [H], dgamma_q [D]."""
    lib = _load()
    qa, qd = _act(q)
    ka, kd = _act(kv_c)
    ra, rd = _act(kv_raw)
    if not (qd == kd == rd):
        raise ValueError("q, kv_c and kv_raw must share one storage type")
    B, Q, H, D = qa.shape
    N, R = ka.shape[1], ra.shape[1]
    ia, K = (None, 0) if idx is None else (_np(idx, np.int32), np.asarray(idx).shape[-1])
    rp, qp, sk = _np(raw_pos0, np.int32), _np(q_pos, np.int32), _np(sinks, np.float32)
    gq = None if gamma_q is None else _np(gamma_q, np.float32)
    gk = None if gamma_kv is None else _np(gamma_kv, np.float32)
    do = _np(dout, np.float32)
    assert do.shape == (B, Q, H, D)
    res = dict(dq=np.empty((B, Q, H, D)), dkhat_c=np.empty((B, N, D)), dkhat_raw=np.empty((B, R, D)),
               dsinks=np.empty((H,)), dgamma_q=np.empty((D,)))
    prm = AttnParams(m, n_win, rope_dims, entry_pos_offset, rope_base, softmax_scale, rms_eps)
    _check(lib.oracle_attention_bwd(ctypes.byref(prm), _ptr(qa), _ptr(ka), _ptr(ia), K, _ptr(ra), _ptr(rp), _ptr(qp),
                                    _ptr(sk), _ptr(gq), _ptr(gk), qd, B, Q, H, D, N, R, _ptr(do), _ptr(res["dq"]),
                                    _ptr(res["dkhat_c"]), _ptr(res["dkhat_raw"]), _ptr(res["dsinks"]),
                                    _ptr(res["dgamma_q"])), "attention_bwd")
    return res
