"""MI355X (gfx950) compressed attention: the DeepSeek-V4 CSA / HCA hot path.

Thin binding over the C ABI of ``libcakv.so`` (include/cakv.h).  Every step
runs in the HIP kernels; this module only marshals torch tensors (device
memory and the current stream) and allocates workspaces.  There is no
fallback: if the library is missing or no GPU is present, calls raise.

Functions (names follow the C ABI):
  kv_compress(x, gate, m, out_dtype)                      -> out (, scale)
  kv_compress_ex(x, gate, m, span, out_dtype)              -> out (, scale)   (overlap, per-channel gates)
  kv_append(x_tok, gate_tok, pos, raw_ring, gate_ring, cache, ...)  streaming decode: one token per sequence
  kv_append_batch([dict of kv_append's arguments, ...], pos)       several of them in one launch
  kv_prepare(kv_c, m, rope_dims, ...)                     -> prepared entries (in place by default)
  kv_prepare_raw(kv_raw, raw_pos0, rope_dims, ...)        -> prepared window rows (per-sequence positions)
  indexer_topk(q_idx, w, k_idx, k_scale, q_pos, m, k)     -> idx
  indexer_topk_noalloc(q_idx, w, k_idx, k_scale, q_pos, m, k, out) -> idx (static scratch)
  sparse_mqa_fwd(q, kv_c, idx, kv_raw, raw_pos0, q_pos, sinks, ...) -> (out, lse)
  dense_compressed_mqa_fwd(q, kv_c, kv_raw, raw_pos0, q_pos, sinks, ...) -> (out, lse)
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcakv.so")

F32, BF16, FP8_E4M3 = 0, 1, 2
_DT = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3, torch.uint8: FP8_E4M3}


class CakvError(RuntimeError):
    pass


class AttnParams(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("n_win", ctypes.c_int32), ("rope_dims", ctypes.c_int32),
                ("rope_base", ctypes.c_float),
                ("softmax_scale", ctypes.c_float), ("rms_eps", ctypes.c_float),
                ("gamma_q", ctypes.c_void_p), ("raw_ring", ctypes.c_int32)]


class PrepParams(ctypes.Structure):
    _fields_ = [("rope_dims", ctypes.c_int32), ("rope_base", ctypes.c_float), ("entry_pos_offset", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("gamma_kv", ctypes.c_void_p)]


class AppendCall(ctypes.Structure):
    """cakv_append_call: one append of a cakv_kv_append_batch."""
    _fields_ = [("x_tok", ctypes.c_void_p), ("gate_tok", ctypes.c_void_p), ("gate_per_channel", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("D", ctypes.c_int64), ("raw_ring", ctypes.c_void_p),
                ("gate_ring", ctypes.c_void_p), ("Rr", ctypes.c_int64), ("win_ring", ctypes.c_void_p),
                ("Rw", ctypes.c_int64), ("cache", ctypes.c_void_p), ("cache_dtype", ctypes.c_int32),
                ("m", ctypes.c_int32), ("cache_scale", ctypes.c_void_p), ("N", ctypes.c_int64),
                ("span", ctypes.c_int32), ("prep", ctypes.POINTER(PrepParams))]


_lib = None
_i64, _i32, _p, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t

EXPORTS = ("cakv_version", "cakv_last_error", "cakv_kv_compress", "cakv_kv_prepare", "cakv_indexer_topk_workspace",
           "cakv_indexer_topk", "cakv_sparse_mqa_workspace", "cakv_sparse_mqa_fwd",
           "cakv_dense_mqa_workspace", "cakv_dense_compressed_mqa_fwd", "cakv_profile_kernel_events",
           "cakv_indexer_topk_noalloc", "cakv_kv_compress_ex", "cakv_kv_append", "cakv_mqa_bwd_workspace",
           "cakv_mqa_bwd", "cakv_kv_prepare_bwd", "cakv_kv_compress_bwd_workspace", "cakv_kv_compress_bwd",
           "cakv_indexer_bwd", "cakv_kv_append_batch")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libcakv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise CakvError(f"{path} is missing: build it first (python -m compressed_attention_kv_amd.build)")
    lib = ctypes.CDLL(path)
    lib.cakv_version.restype = ctypes.c_int
    lib.cakv_last_error.restype = ctypes.c_char_p
    lib.cakv_profile_kernel_events.argtypes = [ctypes.c_char_p, ctypes.POINTER(_p), ctypes.POINTER(_p), ctypes.c_int]
    lib.cakv_kv_compress.argtypes = [_p, ctypes.c_int, _p, _i64, _i64, _i64, _i32, _p, ctypes.c_int, _p, _p]
    lib.cakv_kv_compress_ex.argtypes = [_p, ctypes.c_int, _p, ctypes.c_int, _i64, _i64, _i64, _i32, _i32, _p,
                                        ctypes.c_int, _p, _p]
    lib.cakv_kv_append_batch.argtypes = [ctypes.POINTER(AppendCall), _i32, _p, _i64, _p]
    lib.cakv_kv_append.argtypes = [_p, _p, ctypes.c_int, _p, ctypes.c_int, _i64, _i64, _p, _p, _i64, _p, _i64, _p,
                                   ctypes.c_int, _p, _i64, _i32, _i32, ctypes.POINTER(PrepParams), _p]
    lib.cakv_mqa_bwd_workspace.argtypes = [_i64, _i64, _i32, _i32, _i64, _i32]
    lib.cakv_mqa_bwd_workspace.restype = _sz
    lib.cakv_mqa_bwd.argtypes = [ctypes.POINTER(AttnParams), _p, _p, _p, _p, _p, _p, _p, ctypes.c_int, _i64, _i64,
                                 _i32, _i32, _i64, _i32, _i64, _p, ctypes.c_int, _p, _p, _p, _p, _p, _p, _p, _p, _sz,
                                 _p]
    lib.cakv_kv_prepare_bwd.argtypes = [_p, ctypes.c_int, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _p, _i32, _i32,
                                        ctypes.c_float, _i32, ctypes.c_float, _p]
    lib.cakv_kv_compress_bwd_workspace.argtypes = [_i64, _i64, _i64, _i32]
    lib.cakv_kv_compress_bwd_workspace.restype = _sz
    lib.cakv_kv_compress_bwd.argtypes = [_p, ctypes.c_int, _p, ctypes.c_int, _i64, _i64, _i64, _i32, _i32, _p, _p,
                                         _p, _p, _sz, _p]
    lib.cakv_indexer_bwd.argtypes = [_p, ctypes.c_int, _p, _p, ctypes.c_int, _p, _p, _p, _p, _i64, _i64, _i64, _i32,
                                     _i32, _i32, _i32, _p, _p, _p, _p]
    lib.cakv_kv_prepare.argtypes = [_p, _p, ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _p, _i32, _i32,
                                    ctypes.c_float, _i32, ctypes.c_float, _p]
    lib.cakv_indexer_topk_workspace.argtypes = [_i64, _i64, _i64, _i32]
    lib.cakv_indexer_topk_workspace.restype = _sz
    lib.cakv_indexer_topk.argtypes = [_p, ctypes.c_int, _p, _p, ctypes.c_int, _p, _p, _i64, _i64, _i64, _i32,
                                      _i32, _i32, _i32, _p, _p, _sz, _p]
    lib.cakv_indexer_topk_noalloc.argtypes = [_p, ctypes.c_int, _p, _p, ctypes.c_int, _p, _p, _i64, _i64, _i64,
                                              _i32, _i32, _i32, _i32, _p, _p]
    lib.cakv_sparse_mqa_workspace.argtypes = [_i64, _i64, _i32, _i32, _i32, _i32]
    lib.cakv_sparse_mqa_workspace.restype = _sz
    lib.cakv_dense_mqa_workspace.argtypes = [_i64, _i64, _i32, _i32, _i64, _i32]
    lib.cakv_dense_mqa_workspace.restype = _sz
    lib.cakv_sparse_mqa_fwd.argtypes = [ctypes.POINTER(AttnParams), _p, _p, _p, _p, _p, _p, _p, ctypes.c_int, _i64,
                                        _i64, _i32, _i32, _i64, _i32, _i64, _p, ctypes.c_int, _p, _p, _sz, _p]
    lib.cakv_dense_compressed_mqa_fwd.argtypes = [ctypes.POINTER(AttnParams), _p, _p, _p, _p, _p, _p, ctypes.c_int,
                                                  _i64, _i64, _i32, _i32, _i64, _i64, _p, ctypes.c_int, _p, _p, _sz,
                                                  _p]
    _lib = lib
    return lib


def _check(rc: int):
    if rc != 0:
        raise CakvError(f"cakv error {rc}: {_lib.cakv_last_error().decode()}")


def _dev(t: torch.Tensor | None, name: str, dtype: torch.dtype | None = None):
    """Device pointer of a contiguous device tensor (None -> NULL); with
    `dtype`, the tensor must hold exactly that element type (an int64 position
    tensor, torch's default for integers, would otherwise be read as pairs of
    int32 words)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise CakvError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise CakvError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise CakvError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


_I32, _F32 = torch.int32, torch.float32


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch allocations are 256-byte aligned (512 on ROCm); at least one byte
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def kv_compress(x: torch.Tensor, gate: torch.Tensor, m: int, out_dtype: torch.dtype = None,
                out: torch.Tensor = None, scale: torch.Tensor = None):
    """Softmax-gated compression of every m tokens.  x [B,T,D] f32/bf16, gate [B,T] f32.
    Returns out [B,T//m,D] (out_dtype: float32, bfloat16 or float8_e4m3fn) and, for fp8,
    the per-entry float32 scale [B,T//m].  `out` / `scale` may be given (contiguous,
    e.g. the tail of a cache); they are written in place."""
    lib = load_library()
    B, T, D = x.shape
    out_dtype = out.dtype if out is not None else (out_dtype or x.dtype)
    nb = T // m
    if out is None:
        out = torch.empty((B, nb, D), dtype=out_dtype, device=x.device)
    elif tuple(out.shape) != (B, nb, D) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous [{B}, {nb}, {D}] tensor")
    if out_dtype == torch.float8_e4m3fn and scale is None:
        scale = torch.empty((B, nb), dtype=torch.float32, device=x.device)
    elif out_dtype != torch.float8_e4m3fn:
        scale = None
    _check(lib.cakv_kv_compress(_dev(x, "x"), _DT[x.dtype], _dev(gate, "gate", _F32), B, T, D, m, _dev(out, "out"),
                                _DT[out_dtype], _dev(scale, "scale", _F32), _stream()))
    return (out, scale) if scale is not None else out


def kv_compress_ex(x: torch.Tensor, gate: torch.Tensor, m: int, span: int = None, out_dtype: torch.dtype = None,
                   out: torch.Tensor = None, scale: torch.Tensor = None):
    """Compressor variants: entry j is the softmax-gated sum of the `span`
    tokens ending where block j ends (span >= m); gate [B,T] (one logit per
    token) or [B,T,D] (one per token and channel).  Otherwise as kv_compress."""
    lib = load_library()
    B, T, D = x.shape
    span = m if span is None else span
    per_channel = gate.dim() == 3
    out_dtype = out.dtype if out is not None else (out_dtype or x.dtype)
    nb = T // m
    if out is None:
        out = torch.empty((B, nb, D), dtype=out_dtype, device=x.device)
    elif tuple(out.shape) != (B, nb, D) or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous [{B}, {nb}, {D}] tensor")
    if out_dtype == torch.float8_e4m3fn and scale is None:
        scale = torch.empty((B, nb), dtype=torch.float32, device=x.device)
    elif out_dtype != torch.float8_e4m3fn:
        scale = None
    _check(lib.cakv_kv_compress_ex(_dev(x, "x"), _DT[x.dtype], _dev(gate, "gate", _F32), int(per_channel), B, T, D,
                                   m, span, _dev(out, "out"), _DT[out_dtype], _dev(scale, "scale", _F32), _stream()))
    return (out, scale) if scale is not None else out


def kv_append(x_tok: torch.Tensor, gate_tok: torch.Tensor, pos: torch.Tensor, raw_ring: torch.Tensor,
              gate_ring: torch.Tensor, cache: torch.Tensor, *, m: int, span: int = None,
              cache_scale: torch.Tensor = None, win_ring: torch.Tensor = None, prep: dict | None = None) -> None:
    """One new token per sequence into one compressor's state (see cakv_kv_append):
    x_tok [B,D] at positions pos [B] int32 (-1: none) enters raw_ring [B,Rr,D]
    (gates gate_ring [B,Rr] or [B,Rr,D]), prepared into win_ring [B,Rw,D] if
    given, and a completed block's entry into cache [B,N,D] (prepared with
    `prep` = dict(rope_dims, rope_base, entry_pos_offset, rms_eps, gamma_kv),
    or fp8 codes + cache_scale when prep is None)."""
    lib = load_library()
    B, D = x_tok.shape
    span = m if span is None else span
    per_channel = gate_tok.dim() == 2
    pp = _prep_params(prep)
    if raw_ring.dtype != x_tok.dtype or (win_ring is not None and win_ring.dtype != x_tok.dtype):
        raise CakvError("raw_ring and win_ring must have x_tok's dtype")
    _check(lib.cakv_kv_append(_dev(x_tok, "x_tok"), _dev(gate_tok, "gate_tok", _F32), int(per_channel),
                              _dev(pos, "pos", _I32), _DT[x_tok.dtype], B, D, _dev(raw_ring, "raw_ring"),
                              _dev(gate_ring, "gate_ring", _F32), raw_ring.shape[1], _dev(win_ring, "win_ring"),
                              0 if win_ring is None else win_ring.shape[1], _dev(cache, "cache"), _DT[cache.dtype],
                              _dev(cache_scale, "cache_scale", _F32), cache.shape[1], m, span,
                              None if pp is None else ctypes.byref(pp), _stream()))


def _prep_params(prep: dict | None):
    if prep is None:
        return None
    return PrepParams(int(prep.get("rope_dims", 0)), float(prep.get("rope_base", 10000.0)),
                      int(prep.get("entry_pos_offset", 0)), float(prep.get("rms_eps", 1e-6)),
                      _dev(prep.get("gamma_kv"), "gamma_kv", _F32))


def kv_append_batch(calls, pos: torch.Tensor) -> None:
    """Several appends of the same new tokens (positions pos [B] int32) in one
    launch (see cakv_kv_append_batch): each element of `calls` is a dict of
    kv_append's arguments -- x_tok, gate_tok, raw_ring, gate_ring, cache, m,
    and optionally span, cache_scale, win_ring, prep.  The results are those
    of the same kv_append calls made one after another."""
    lib = load_library()
    n = len(calls)
    B = pos.shape[0]
    arr = (AppendCall * max(n, 1))()
    preps = []  # the PrepParams stay referenced until the call returns
    for i, c in enumerate(calls):
        x, g, raw, graw, cache = c["x_tok"], c["gate_tok"], c["raw_ring"], c["gate_ring"], c["cache"]
        win, cs = c.get("win_ring"), c.get("cache_scale")
        if x.shape[0] != B:
            raise CakvError(f"kv_append_batch: append {i} has {x.shape[0]} tokens, pos has {B}")
        if raw.dtype != x.dtype or (win is not None and win.dtype != x.dtype):
            raise CakvError("raw_ring and win_ring must have x_tok's dtype")
        pp = _prep_params(c.get("prep"))
        preps.append(pp)
        m = int(c["m"])
        arr[i] = AppendCall(_dev(x, "x_tok"), _dev(g, "gate_tok", _F32), int(g.dim() == 2), _DT[x.dtype], x.shape[1],
                            _dev(raw, "raw_ring"), _dev(graw, "gate_ring", _F32), raw.shape[1], _dev(win, "win_ring"),
                            0 if win is None else win.shape[1], _dev(cache, "cache"), _DT[cache.dtype], m,
                            _dev(cs, "cache_scale", _F32), cache.shape[1], int(c.get("span") or m),
                            None if pp is None else ctypes.pointer(pp))
    _check(lib.cakv_kv_append_batch(arr, n, _dev(pos, "pos", _I32), B, _stream()))


def kv_prepare(kv_c: torch.Tensor, *, m: int, rope_dims: int, rope_base: float = 10000.0,
               entry_pos_offset: int = 0, rms_eps: float = 1e-6, gamma_kv=None, j0: int = 0, n: int = None,
               out: torch.Tensor = None) -> torch.Tensor:
    """Key/value vectors of compressed entries j0 .. j0+n-1 (all by default) of kv_c [B,N,D]
    (f32/bf16): RMSNorm with gamma_kv, the last rope_dims dims rotated by j*m + entry_pos_offset.
    Written into `out` (same shape) or, by default, in place into kv_c; returns it.  The
    attention calls read compressed entries in this form."""
    lib = load_library()
    B, N, D = kv_c.shape
    n = N - j0 if n is None else n
    out = kv_c if out is None else out
    if tuple(out.shape) != (B, N, D) or out.dtype != kv_c.dtype:
        raise ValueError("out must match kv_c in shape and dtype")
    _check(lib.cakv_kv_prepare(_dev(kv_c, "kv_c"), _dev(out, "out"), _DT[kv_c.dtype], B, N, D, j0, n,
                               _dev(gamma_kv, "gamma_kv", _F32), m, rope_dims, rope_base, entry_pos_offset, rms_eps,
                               _stream()))
    return out


def kv_prepare_raw(kv_raw: torch.Tensor, raw_pos0, *, rope_dims: int, rope_base: float = 10000.0,
                   rms_eps: float = 1e-6, gamma_kv=None, out: torch.Tensor = None) -> torch.Tensor:
    """Window rows of kv_raw [B,R,D] prepared at their positions raw_pos0[b] + r
    (kv_prepare with m = 1, one call per sequence); raw_pos0 is a host sequence of B ints."""
    out = kv_raw if out is None else out
    for b, p0 in enumerate(int(v) for v in raw_pos0):
        kv_prepare(kv_raw[b:b + 1], m=1, rope_dims=rope_dims, rope_base=rope_base, entry_pos_offset=p0,
                   rms_eps=rms_eps, gamma_kv=gamma_kv, out=out[b:b + 1])
    return out


def indexer_topk_workspace_bytes(B: int, Q: int, N: int, k: int) -> int:
    return int(load_library().cakv_indexer_topk_workspace(B, Q, N, k))


def indexer_topk(q_idx: torch.Tensor, w: torch.Tensor, k_idx: torch.Tensor, k_scale: torch.Tensor | None,
                 q_pos: torch.Tensor, m: int, k: int, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Top-k compressed entries per query: idx [B,Q,k] int32, ascending, -1 padded.
    Modes: (q f32, k f32) canonical fp32; (q bf16, k fp8 + k_scale) matrix-core."""
    lib = load_library()
    B, Q, HI, dI = q_idx.shape
    N = k_idx.shape[1]
    if out is None:
        out = torch.empty((B, Q, k), dtype=torch.int32, device=q_idx.device)
    need = int(lib.cakv_indexer_topk_workspace(B, Q, N, k))
    if workspace is None or workspace.numel() < need:
        workspace = _workspace(need, q_idx.device)
    _check(lib.cakv_indexer_topk(_dev(q_idx, "q_idx"), _DT[q_idx.dtype], _dev(w, "w", _F32), _dev(k_idx, "k_idx"),
                                 _DT[k_idx.dtype], _dev(k_scale, "k_scale", _F32), _dev(q_pos, "q_pos", _I32), B, Q, N, HI, dI,
                                 m, k, _dev(out, "idx", _I32), workspace.data_ptr(), workspace.numel(), _stream()))
    return out


def _same_act(q, kv_c, kv_raw):
    # the C ABI takes one activation type for q, the cache and the window rows
    if not (q.dtype == kv_c.dtype == kv_raw.dtype):
        raise CakvError(f"q, kv_c and kv_raw must share one dtype ({q.dtype}, {kv_c.dtype}, {kv_raw.dtype})")


def indexer_topk_noalloc(q_idx: torch.Tensor, w: torch.Tensor, k_idx: torch.Tensor, k_scale: torch.Tensor | None,
                         q_pos: torch.Tensor, m: int, k: int, out: torch.Tensor) -> torch.Tensor:
    """indexer_topk into a caller-provided `out` [B,Q,k] int32, with the
    library's static per-GPU scratch as its workspace (no device allocation
    by the library or here)."""
    lib = load_library()
    B, Q, HI, dI = q_idx.shape
    N = k_idx.shape[1]
    if tuple(out.shape) != (B, Q, k):
        raise CakvError(f"out must be [{B}, {Q}, {k}]")
    _check(lib.cakv_indexer_topk_noalloc(_dev(q_idx, "q_idx"), _DT[q_idx.dtype], _dev(w, "w", _F32),
                                         _dev(k_idx, "k_idx"), _DT[k_idx.dtype], _dev(k_scale, "k_scale", _F32),
                                         _dev(q_pos, "q_pos", _I32), B, Q, N, HI, dI, m, k, _dev(out, "idx", _I32),
                                         _stream()))
    return out


def _params(m, n_win, rope_dims, rope_base, softmax_scale, rms_eps, gamma_q, raw_ring=False):
    return AttnParams(m, n_win, rope_dims, rope_base, softmax_scale, rms_eps, _dev(gamma_q, "gamma_q", _F32),
                      int(bool(raw_ring)))


def sparse_mqa_workspace_bytes(B, Q, H, D, K, n_win) -> int:
    return int(load_library().cakv_sparse_mqa_workspace(B, Q, H, D, K, n_win))


def dense_mqa_workspace_bytes(B, Q, H, D, N, n_win) -> int:
    return int(load_library().cakv_dense_mqa_workspace(B, Q, H, D, N, n_win))


def sparse_mqa_fwd(q, kv_c, idx, kv_raw, raw_pos0, q_pos, sinks, *, m: int, n_win: int, rope_dims: int,
                   rope_base: float = 10000.0, softmax_scale: float = 0.0,
                   rms_eps: float = 1e-6, gamma_q=None, out_dtype=None, want_lse=True,
                   out=None, workspace=None, raw_ring: bool = False):
    """CSA core attention over the selected entries + raw window + sink.
    q [B,Q,H,D], kv_c [B,N,D], idx [B,Q,K] int32, kv_raw [B,R,D]; returns (out, lse).
    kv_c and kv_raw hold rows prepared by kv_prepare (raw row r of sequence b at
    position raw_pos0[b] + r: kv_prepare_raw), or, with raw_ring=True, kv_raw is
    the window ring kv_append keeps (row p mod R holds position p; raw_pos0 may
    be None)."""
    lib = load_library()
    B, Q, H, D = q.shape
    N, R, K = kv_c.shape[1], kv_raw.shape[1], idx.shape[-1]
    _same_act(q, kv_c, kv_raw)
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, Q, H, D), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=q.device) if want_lse else None
    need = int(lib.cakv_sparse_mqa_workspace(B, Q, H, D, K, n_win))
    if workspace is None or workspace.numel() < need:
        workspace = _workspace(need, q.device)
    prm = _params(m, n_win, rope_dims, rope_base, softmax_scale, rms_eps, gamma_q, raw_ring)
    _check(lib.cakv_sparse_mqa_fwd(ctypes.byref(prm), _dev(q, "q"), _dev(kv_c, "kv_c"), _dev(idx, "idx", _I32),
                                   _dev(kv_raw, "kv_raw"), _dev(raw_pos0, "raw_pos0", _I32), _dev(q_pos, "q_pos", _I32),
                                   _dev(sinks, "sinks", _F32), _DT[q.dtype], B, Q, H, D, N, K, R, _dev(out, "out"),
                                   _DT[out_dtype], _dev(lse, "lse", _F32), workspace.data_ptr(), workspace.numel(),
                                   _stream()))
    return out, lse


def dense_compressed_mqa_fwd(q, kv_c, kv_raw, raw_pos0, q_pos, sinks, *, m: int, n_win: int, rope_dims: int,
                             rope_base: float = 10000.0, softmax_scale: float = 0.0,
                             rms_eps: float = 1e-6, gamma_q=None, out_dtype=None, want_lse=True,
                             out=None, workspace=None, raw_ring: bool = False):
    """HCA core attention over every visible compressed entry + raw window + sink
    (rows prepared as for sparse_mqa_fwd)."""
    lib = load_library()
    B, Q, H, D = q.shape
    N, R = kv_c.shape[1], kv_raw.shape[1]
    _same_act(q, kv_c, kv_raw)
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, Q, H, D), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=q.device) if want_lse else None
    need = int(lib.cakv_dense_mqa_workspace(B, Q, H, D, N, n_win))
    if workspace is None or workspace.numel() < need:
        workspace = _workspace(need, q.device)
    prm = _params(m, n_win, rope_dims, rope_base, softmax_scale, rms_eps, gamma_q, raw_ring)
    _check(lib.cakv_dense_compressed_mqa_fwd(ctypes.byref(prm), _dev(q, "q"), _dev(kv_c, "kv_c"),
                                             _dev(kv_raw, "kv_raw"), _dev(raw_pos0, "raw_pos0", _I32),
                                             _dev(q_pos, "q_pos", _I32), _dev(sinks, "sinks", _F32), _DT[q.dtype], B, Q, H, D,
                                             N, R, _dev(out, "out"), _DT[out_dtype], _dev(lse, "lse", _F32),
                                             workspace.data_ptr(), workspace.numel(), _stream()))
    return out, lse


def version() -> int:
    return int(load_library().cakv_version())


def profile_kernel_events(kernel: str | None, starts=(), ends=()) -> None:
    """Profiling aid: the library records the given torch.cuda.Event pairs around
    the next len(starts) launches of `kernel` made from this thread (None clears).
    The events are created here if they have not been recorded yet."""
    lib = load_library()
    n = len(starts)
    if kernel is None or n == 0:
        _check(lib.cakv_profile_kernel_events(None, None, None, 0))
        return
    for e in list(starts) + list(ends):
        if e.cuda_event == 0:
            e.record()
    arr = (_p * n)
    _check(lib.cakv_profile_kernel_events(kernel.encode(), arr(*[e.cuda_event for e in starts]),
                                          arr(*[e.cuda_event for e in ends]), n))


# ---------------------------------------------------------------- backward (training)

def mqa_bwd(q, kv_c, idx, kv_raw, raw_pos0, q_pos, sinks, out, lse, dout, *, m: int, n_win: int, rope_dims: int,
            rope_base: float = 10000.0, softmax_scale: float = 0.0, rms_eps: float = 1e-6, gamma_q=None,
            raw_ring: bool = False, dkv_c=None, dkv_raw=None, dsinks=None, dgamma_q=None, workspace=None):
    """Gradient of sparse_mqa_fwd (idx given) or dense_compressed_mqa_fwd (idx
    None) from the forward's inputs, out, lse and dout [B,Q,H,D] float32.
    Returns dict(dq, dkv_c, dkv_raw, dsinks, dgamma_q): dq is new; the others
    are accumulated into the given float32 tensors (zero-filled new ones by
    default; dgamma_q only when gamma_q is given).  dkv_c / dkv_raw are the
    gradients of the prepared rows (kv_prepare_bwd continues to raw rows)."""
    lib = load_library()
    B, Q, H, D = q.shape
    N, R = kv_c.shape[1], kv_raw.shape[1]
    K = idx.shape[-1] if idx is not None else 0
    _same_act(q, kv_c, kv_raw)
    dev = q.device
    dq = torch.empty((B, Q, H, D), dtype=torch.float32, device=dev)
    dkv_c = torch.zeros((B, N, D), dtype=torch.float32, device=dev) if dkv_c is None else dkv_c
    dkv_raw = torch.zeros((B, R, D), dtype=torch.float32, device=dev) if dkv_raw is None else dkv_raw
    dsinks = torch.zeros((H,), dtype=torch.float32, device=dev) if dsinks is None else dsinks
    if gamma_q is not None and dgamma_q is None:
        dgamma_q = torch.zeros((D,), dtype=torch.float32, device=dev)
    n_keys = K if idx is not None else N
    need = int(lib.cakv_mqa_bwd_workspace(B, Q, H, D, n_keys, n_win))
    if workspace is None or workspace.numel() < need:
        workspace = _workspace(need, dev)
    prm = _params(m, n_win, rope_dims, rope_base, softmax_scale, rms_eps, gamma_q, raw_ring)
    _check(lib.cakv_mqa_bwd(ctypes.byref(prm), _dev(q, "q"), _dev(kv_c, "kv_c"), _dev(idx, "idx", _I32),
                            _dev(kv_raw, "kv_raw"), _dev(raw_pos0, "raw_pos0", _I32), _dev(q_pos, "q_pos", _I32),
                            _dev(sinks, "sinks", _F32), _DT[q.dtype], B, Q, H, D, N, K, R, _dev(out, "out"),
                            _DT[out.dtype], _dev(lse, "lse", _F32), _dev(dout, "dout", _F32), _dev(dq, "dq", _F32),
                            _dev(dkv_c, "dkv_c", _F32), _dev(dkv_raw, "dkv_raw", _F32), _dev(dsinks, "dsinks", _F32),
                            _dev(dgamma_q, "dgamma_q", _F32), workspace.data_ptr(), workspace.numel(), _stream()))
    return dict(dq=dq, dkv_c=dkv_c, dkv_raw=dkv_raw, dsinks=dsinks, dgamma_q=dgamma_q)


def kv_prepare_bwd(kv_in, dy, *, m: int, rope_dims: int, rope_base: float = 10000.0, entry_pos_offset: int = 0,
                   rms_eps: float = 1e-6, gamma_kv=None, j0: int = 0, n: int = None, dx=None, dgamma_kv=None):
    """Gradient of kv_prepare: dy [B,N,D] float32 of the prepared rows ->
    dx [B,N,D] float32 of the raw entries (rows j0 .. j0+n-1; a new zero
    tensor by default) and dgamma_kv (accumulated when given).  Returns dx."""
    lib = load_library()
    B, N, D = kv_in.shape
    n = N - j0 if n is None else n
    dx = torch.zeros((B, N, D), dtype=torch.float32, device=kv_in.device) if dx is None else dx
    _check(lib.cakv_kv_prepare_bwd(_dev(kv_in, "kv_in"), _DT[kv_in.dtype], _dev(dy, "dy", _F32), _dev(dx, "dx", _F32),
                                   _dev(dgamma_kv, "dgamma_kv", _F32), B, N, D, j0, n,
                                   _dev(gamma_kv, "gamma_kv", _F32), m, rope_dims, rope_base, entry_pos_offset,
                                   rms_eps, _stream()))
    return dx


def kv_compress_bwd(x, gate, m: int, dc, span: int = None):
    """Gradient of kv_compress_ex: dc [B,T//m,D] float32 -> (dx [B,T,D],
    dgate of gate's shape), float32."""
    lib = load_library()
    B, T, D = x.shape
    span = m if span is None else span
    per_channel = gate.dim() == 3
    dx = torch.empty((B, T, D), dtype=torch.float32, device=x.device)
    dg = torch.empty(gate.shape, dtype=torch.float32, device=x.device)
    need = int(lib.cakv_kv_compress_bwd_workspace(B, T, D, m))
    ws = _workspace(need, x.device)
    _check(lib.cakv_kv_compress_bwd(_dev(x, "x"), _DT[x.dtype], _dev(gate, "gate", _F32), int(per_channel), B, T, D,
                                    m, span, _dev(dc, "dc", _F32), _dev(dx, "dx", _F32), _dev(dg, "dgate", _F32),
                                    ws.data_ptr(), ws.numel(), _stream()))
    return dx, dg


def indexer_bwd(q_idx, w, k_idx, k_scale, q_pos, idx, dS, m: int, dk=None):
    """Gradient of the indexer score over the selected entries idx [B,Q,K]
    given dS [B,Q,K] float32 -> (dq_idx [B,Q,HI,dI], dw [B,Q,HI], dk
    [B,N,dI] accumulated; new zero tensor by default), float32."""
    lib = load_library()
    B, Q, HI, dI = q_idx.shape
    N, K = k_idx.shape[1], idx.shape[-1]
    dq = torch.empty((B, Q, HI, dI), dtype=torch.float32, device=q_idx.device)
    dw = torch.empty((B, Q, HI), dtype=torch.float32, device=q_idx.device)
    dk = torch.zeros((B, N, dI), dtype=torch.float32, device=q_idx.device) if dk is None else dk
    _check(lib.cakv_indexer_bwd(_dev(q_idx, "q_idx"), _DT[q_idx.dtype], _dev(w, "w", _F32), _dev(k_idx, "k_idx"),
                                _DT[k_idx.dtype], _dev(k_scale, "k_scale", _F32), _dev(q_pos, "q_pos", _I32),
                                _dev(idx, "idx", _I32), _dev(dS, "dS", _F32), B, Q, N, HI, dI, m, K,
                                _dev(dq, "dq_idx", _F32), _dev(dw, "dw", _F32), _dev(dk, "dk", _F32), _stream()))
    return dq, dw, dk


# ---------------------------------------------------------------- measurement probes (include/cakv_probes.h)

PROBES_PATH = os.path.join(_HERE, "libcakv_probes.so")
PROBE_EXPORTS = ("cakv_probe_read", "cakv_probe_mfma_bf16")
_probes = None


def load_probes(path: str = PROBES_PATH) -> ctypes.CDLL:
    """Load libcakv_probes.so, the attainable-peak probes (built with the library)."""
    global _probes
    if _probes is not None:
        return _probes
    if not os.path.exists(path):
        raise CakvError(f"{path} is missing: build it first (python -m compressed_attention_kv_amd.build)")
    lib = ctypes.CDLL(path)
    lib.cakv_probe_read.argtypes = [_p, _sz, _p, _i32, _p]
    lib.cakv_probe_read.restype = ctypes.c_int
    lib.cakv_probe_mfma_bf16.argtypes = [_i64, _i32, _p, _p]
    lib.cakv_probe_mfma_bf16.restype = ctypes.c_int
    _probes = lib
    return lib


def probe_read(buf: torch.Tensor, sink: torch.Tensor, blocks: int = 0) -> None:
    """Streaming read of every byte of `buf` (contiguous, on the GPU, a
    multiple of 16 bytes); workgroup g writes the XOR of the 32-bit words it
    read to sink[g] (int32, at least `blocks` elements; blocks 0 means 2048)."""
    lib = load_probes()
    if not (buf.is_cuda and buf.is_contiguous() and sink.is_cuda and sink.is_contiguous()):
        raise CakvError("probe_read: buf and sink must be contiguous tensors on the GPU")
    if sink.dtype != torch.int32 or sink.numel() < (blocks or 2048):
        raise CakvError("probe_read: sink must be int32 with one element per workgroup")
    rc = lib.cakv_probe_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), blocks, _stream())
    if rc != 0:
        raise CakvError(f"cakv_probe_read returned {rc}")


def probe_mfma_bf16(iters: int, blocks: int, sink: torch.Tensor) -> float:
    """The bf16 MFMA loop: `blocks` workgroups of four waves, `iters` rounds
    of four independent 32x32x16 MFMAs per wave; sink (float32, 4 * blocks)
    gets one sum per wave.  Returns the flops the launch performs."""
    lib = load_probes()
    if not (sink.is_cuda and sink.is_contiguous() and sink.dtype == torch.float32 and sink.numel() >= 4 * blocks):
        raise CakvError("probe_mfma_bf16: sink must be a contiguous float32 GPU tensor of 4 * blocks elements")
    rc = lib.cakv_probe_mfma_bf16(iters, blocks, sink.data_ptr(), _stream())
    if rc != 0:
        raise CakvError(f"cakv_probe_mfma_bf16 returned {rc}")
    return float(blocks) * 4 * iters * 4 * 32768
