"""Seeded synthetic inputs for the compressed-attention hot path.

This module only draws random numbers and lays them out in the shapes of the
workloads; it contains none of the method's arithmetic (no compression, no
quantisation, no scoring, no attention).  Both the HIP path and the CPU
oracle consume what it returns, so the two sides always see identical bytes.

Every tensor comes from its own child of ``numpy.random.SeedSequence(seed)``,
spawned in a fixed order, drawn as float32 ``standard_normal`` and then cast
to the storage type (bf16 casts use torch's round-to-nearest-even).
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import Workload, get_workload


def _rng_children(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _normal(rng: np.random.Generator, shape, dtype: torch.dtype) -> torch.Tensor:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    t = torch.from_numpy(a)
    return t if dtype == torch.float32 else t.to(dtype)


# Fixed draw order.  Adding a field appends to the end so earlier draws never move.
_FIELDS = ("q", "kv", "gate", "k_idx", "k_gate", "q_idx", "w", "sinks", "kv_raw",
           "hca_gate", "q_hca", "sinks_hca")


def make_inputs(w: Workload | str, only=None, **overrides) -> dict:
    """Return a dict of CPU tensors for workload ``w`` (a name or a Workload).

    ``only``: optional set of field names to draw (others are skipped; every
    field has its own random stream, so skipping never changes the rest).

    Keys (present when the workload uses them):
      q       [B,Q,H,D]   query heads (before norm / rotation)
      kv      decode: compressed KV cache [B,N,D];  prefill: raw KV tokens [B,T,D]
      gate    [B,T]       compressor gate logits for ``kv`` (prefill only)
      k_idx   decode: compressed indexer keys [B,N,dI] (float32, before fp8);
              prefill: raw indexer keys [B,T,dI]
      k_gate  [B,T]       compressor gate logits for ``k_idx`` (prefill only)
      q_idx   [B,Q,HI,dI] indexer queries
      w       [B,Q,HI]    indexer head weights (float32)
      sinks   [H]         per-head sink logits (float32)
      kv_raw  [B,R,D]     raw (uncompressed) KV rows for the sliding window
      raw_pos0 [B]        absolute position of kv_raw row 0 (int32)
      q_pos   [B,Q]       absolute query positions (int32)
      hca_gate, q_hca, sinks_hca   the HCA layer's own gate, queries and sinks (prefill)
    """
    if isinstance(w, str):
        w = get_workload(w, **overrides)
    elif overrides:
        w = w.replace(**overrides)
    rngs = dict(zip(_FIELDS, _rng_children(w.seed, len(_FIELDS))))
    act = torch.float32 if w.dtype == "f32" else torch.bfloat16

    def draw(field, shape, dtype):
        if only is not None and field not in only:
            return None
        return _normal(rngs[field], shape, dtype)

    B, Q, H, D = w.B, w.Q, w.H, w.D
    out: dict = {"workload": w}
    out["q"] = draw("q", (B, Q, H, D), act)
    if w.prefill:
        T = w.T
        out["kv"] = draw("kv", (B, T, D), act)
        out["gate"] = draw("gate", (B, T), torch.float32)
        if w.csa:
            out["k_idx"] = draw("k_idx", (B, T, w.dI), act)
            out["k_gate"] = draw("k_gate", (B, T), torch.float32)
        if w.hca:
            out["hca_gate"] = draw("hca_gate", (B, T), torch.float32)
            out["q_hca"] = draw("q_hca", (B, Q, H, D), act)
            out["sinks_hca"] = draw("sinks_hca", (H,), torch.float32)
        # the raw window source is the raw KV itself: row p holds position p
        out["kv_raw"] = out["kv"]
        out["raw_pos0"] = torch.zeros(B, dtype=torch.int32)
        out["q_pos"] = (w.q_pos0 + torch.arange(Q, dtype=torch.int32)).repeat(B, 1)
    else:
        N = w.N
        out["kv"] = draw("kv", (B, N, D), act)
        if w.csa:
            out["k_idx"] = draw("k_idx", (B, N, w.dI), torch.float32)
        R = w.n_win
        out["kv_raw"] = draw("kv_raw", (B, R, D), act)
        out["q_pos"] = torch.full((B, Q), w.t, dtype=torch.int32)
        out["raw_pos0"] = torch.full((B,), w.t - R + 1, dtype=torch.int32)
    if w.csa:
        out["q_idx"] = draw("q_idx", (B, Q, w.HI, w.dI), act)
        out["w"] = draw("w", (B, Q, w.HI), torch.float32)
    out["sinks"] = draw("sinks", (H,), torch.float32)
    return out
