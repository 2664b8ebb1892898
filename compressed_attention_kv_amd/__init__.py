"""MI355X (gfx950) compressed attention: the DeepSeek-V4 CSA / HCA hot path.

Thin binding over the C ABI of ``libcakv.so`` (include/cakv.h).  Every step
runs in the HIP kernels; this module only marshals torch tensors (device
memory and the current stream) and allocates workspaces.  There is no
fallback: if the library is missing or no GPU is present, calls raise.

Functions (names follow the C ABI):
  kv_compress(x, gate, m, out_dtype)                      -> out (, scale)
  kv_prepare(kv_c, m, rope_dims, ...)                     -> prepared entries (in place by default)
  kv_prepare_raw(kv_raw, raw_pos0, rope_dims, ...)        -> prepared window rows (per-sequence positions)
  indexer_topk(q_idx, w, k_idx, k_scale, q_pos, m, k)     -> idx
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
                ("gamma_q", ctypes.c_void_p)]


_lib = None
_i64, _i32, _p, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t

EXPORTS = ("cakv_version", "cakv_last_error", "cakv_kv_compress", "cakv_kv_prepare", "cakv_indexer_topk_workspace",
           "cakv_indexer_topk", "cakv_sparse_mqa_workspace", "cakv_sparse_mqa_fwd",
           "cakv_dense_mqa_workspace", "cakv_dense_compressed_mqa_fwd", "cakv_profile_kernel_events")


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
    lib.cakv_kv_prepare.argtypes = [_p, _p, ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _p, _i32, _i32,
                                    ctypes.c_float, _i32, ctypes.c_float, _p]
    lib.cakv_indexer_topk_workspace.argtypes = [_i64, _i64, _i64, _i32]
    lib.cakv_indexer_topk_workspace.restype = _sz
    lib.cakv_indexer_topk.argtypes = [_p, ctypes.c_int, _p, _p, ctypes.c_int, _p, _p, _i64, _i64, _i64, _i32,
                                      _i32, _i32, _i32, _p, _p, _sz, _p]
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


def _dev(t: torch.Tensor | None, name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise CakvError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise CakvError(f"{name} must be contiguous")
    return t.data_ptr()


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
    _check(lib.cakv_kv_compress(_dev(x, "x"), _DT[x.dtype], _dev(gate, "gate"), B, T, D, m, _dev(out, "out"),
                                _DT[out_dtype], _dev(scale, "scale"), _stream()))
    return (out, scale) if scale is not None else out


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
                               _dev(gamma_kv, "gamma_kv"), m, rope_dims, rope_base, entry_pos_offset, rms_eps,
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
    _check(lib.cakv_indexer_topk(_dev(q_idx, "q_idx"), _DT[q_idx.dtype], _dev(w, "w"), _dev(k_idx, "k_idx"),
                                 _DT[k_idx.dtype], _dev(k_scale, "k_scale"), _dev(q_pos, "q_pos"), B, Q, N, HI, dI,
                                 m, k, _dev(out, "idx"), workspace.data_ptr(), workspace.numel(), _stream()))
    return out


def _params(m, n_win, rope_dims, rope_base, softmax_scale, rms_eps, gamma_q):
    return AttnParams(m, n_win, rope_dims, rope_base, softmax_scale, rms_eps, _dev(gamma_q, "gamma_q"))


def sparse_mqa_workspace_bytes(B, Q, H, D, K, n_win) -> int:
    return int(load_library().cakv_sparse_mqa_workspace(B, Q, H, D, K, n_win))


def dense_mqa_workspace_bytes(B, Q, H, D, N, n_win) -> int:
    return int(load_library().cakv_dense_mqa_workspace(B, Q, H, D, N, n_win))


def sparse_mqa_fwd(q, kv_c, idx, kv_raw, raw_pos0, q_pos, sinks, *, m: int, n_win: int, rope_dims: int,
                   rope_base: float = 10000.0, softmax_scale: float = 0.0,
                   rms_eps: float = 1e-6, gamma_q=None, out_dtype=None, want_lse=True,
                   out=None, workspace=None):
    """CSA core attention over the selected entries + raw window + sink.
    q [B,Q,H,D], kv_c [B,N,D], idx [B,Q,K] int32, kv_raw [B,R,D]; returns (out, lse).
    kv_c and kv_raw hold rows prepared by kv_prepare (raw row r of sequence b at
    position raw_pos0[b] + r: kv_prepare_raw)."""
    lib = load_library()
    B, Q, H, D = q.shape
    N, R, K = kv_c.shape[1], kv_raw.shape[1], idx.shape[-1]
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, Q, H, D), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=q.device) if want_lse else None
    need = int(lib.cakv_sparse_mqa_workspace(B, Q, H, D, K, n_win))
    if workspace is None or workspace.numel() < need:
        workspace = _workspace(need, q.device)
    prm = _params(m, n_win, rope_dims, rope_base, softmax_scale, rms_eps, gamma_q)
    _check(lib.cakv_sparse_mqa_fwd(ctypes.byref(prm), _dev(q, "q"), _dev(kv_c, "kv_c"), _dev(idx, "idx"),
                                   _dev(kv_raw, "kv_raw"), _dev(raw_pos0, "raw_pos0"), _dev(q_pos, "q_pos"),
                                   _dev(sinks, "sinks"), _DT[q.dtype], B, Q, H, D, N, K, R, _dev(out, "out"),
                                   _DT[out_dtype], _dev(lse, "lse"), workspace.data_ptr(), workspace.numel(),
                                   _stream()))
    return out, lse


def dense_compressed_mqa_fwd(q, kv_c, kv_raw, raw_pos0, q_pos, sinks, *, m: int, n_win: int, rope_dims: int,
                             rope_base: float = 10000.0, softmax_scale: float = 0.0,
                             rms_eps: float = 1e-6, gamma_q=None, out_dtype=None, want_lse=True,
                             out=None, workspace=None):
    """HCA core attention over every visible compressed entry + raw window + sink
    (rows prepared as for sparse_mqa_fwd)."""
    lib = load_library()
    B, Q, H, D = q.shape
    N, R = kv_c.shape[1], kv_raw.shape[1]
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, Q, H, D), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, Q, H), dtype=torch.float32, device=q.device) if want_lse else None
    need = int(lib.cakv_dense_mqa_workspace(B, Q, H, D, N, n_win))
    if workspace is None or workspace.numel() < need:
        workspace = _workspace(need, q.device)
    prm = _params(m, n_win, rope_dims, rope_base, softmax_scale, rms_eps, gamma_q)
    _check(lib.cakv_dense_compressed_mqa_fwd(ctypes.byref(prm), _dev(q, "q"), _dev(kv_c, "kv_c"),
                                             _dev(kv_raw, "kv_raw"), _dev(raw_pos0, "raw_pos0"),
                                             _dev(q_pos, "q_pos"), _dev(sinks, "sinks"), _DT[q.dtype], B, Q, H, D,
                                             N, R, _dev(out, "out"), _DT[out_dtype], _dev(lse, "lse"),
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
