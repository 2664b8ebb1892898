"""Throughput of the compressed-attention hot path on one MI355X.

Headline workload (the line's top-level figures): CSA decode at 128K context
-- 32 sequences, each query at position 131072 over 32768 compressed entries
(m=4) with fp8 indexer keys, top-1024 selection, then sparse MQA (128 heads x
512) over the selection plus the 128-token raw window and the sinks.  One step
= indexer_topk + sparse_mqa_fwd for the batch, inputs resident in HBM, and
the CPU oracle timed beside it on a bounded sample.

With --extras all (the default) every other workload is measured too and
reported under "workloads" (same fields, no CPU baseline):
  csa_decode_1m, hca_decode_1m (dense_compressed_mqa_fwd only),
  prefill_chunk_256k (CSA + HCA layers of an 8192-token chunk after a
    262,144-token prefix: the chunk's compressions and preparations, the
    indexer, sparse attention, dense attention),
  flash_csa_decode_128k, flash_hca_decode_1m (64 heads, top-512),
  stream_decode_128k (the per-token decode step: one batched kv_append of
    the new token into the CSA, indexer-key and HCA state, then indexer and
    both attention calls reading the window rings),
  compress_variants_256k (kv_compress_ex: spans of 8 at m = 4 with
    per-channel gates over a 262,144-token prefix),
  backward_csa_decode_128k (training: mqa_bwd + indexer_bwd at the CSA 128K
    decode shapes).
Decode caches and window rows hold prepared keys (kv_prepare runs once per
entry or token, when it is written).  Decode steps cycle through several
copies of the caches so that the 256 MiB Infinity Cache cannot hold a
step's working set between steps.

Each workload reports its roofline: the dominant kernel's launches timed
with HIP events recorded by the library around that kernel inside the timed
region (less the latency of an empty event pair; the raw figure and, when a
committed rocprofv3 summary of the same sources exists, its mean duration
are listed beside it), the whole step's roofline fraction, and a per-call
breakdown from a separate untimed pass.  --gpus N with N > 1 is not
supported: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import compressed_attention_kv_amd as cakv  # noqa: E402
from compressed_attention_kv_amd.gen import make_inputs  # noqa: E402

METRIC = "CSA/HCA query-tokens/s at 128K-1M ctx; % of HBM BW and MFMA peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFS = 2500.0
FP32_VALU_PEAK_TFS = 157.3
CACHE_BYTES = 256 << 20


def _nvis(w, t) -> int:
    return min(t // w.m, w.N) if w.N else t // w.m


# ---------------------------------------------------------------- algorithmic work per query
def _indexer_score(w, nv: int):
    """bytes, flops of scoring one query: fp8 keys + scales of every visible
    entry, the indexer query heads (bf16) and head weights (f32)."""
    return nv * w.dI + nv * 4 + w.HI * w.dI * 2 + w.HI * 4, 2 * w.HI * w.dI * nv


def _attention(w, rows: int, sparse: bool):
    """bytes, flops of one query's attention: the key rows (bf16), q, the
    output, the indices and the sinks; QK and PV products."""
    return rows * w.D * 2 + 2 * w.H * w.D * 2 + (w.k * 4 if sparse else 0) + w.H * 4, 4 * w.H * w.D * rows


class Step:
    """Device-resident inputs and one step of the path for a workload."""

    def __init__(self, name: str):
        self.name = name
        self.prefill = name.startswith("prefill")
        self.i = 0
        (self._init_prefill if self.prefill else self._init_decode)(name)

    # ------------------------------------------------------------ decode
    def _init_decode(self, name):
        inp = make_inputs(name)
        w = self.w = inp["workload"]
        dev = "cuda"
        self.sparse = w.csa
        nq = w.B * w.Q
        nv = _nvis(w, w.t)
        if self.sparse:
            # the indexer key cache in fp8 + per-entry scale: kv_compress with
            # m = 1 is exactly the per-entry quantiser
            kf = inp["k_idx"].to(dev)
            codes, scale = cakv.kv_compress(kf, torch.zeros(kf.shape[:2], dtype=torch.float32, device=dev), 1,
                                            out_dtype=torch.float8_e4m3fn)
            del kf
            b_s, f_s = _indexer_score(w, nv)
            b_a, f_a = _attention(w, w.k + w.n_win, True)
            step_bytes = (b_s + b_a) * nq
            # kernel -> (algorithmic bytes, flops) per launch
            self.kernels = {"idx_score_fp8_kernel": (b_s * nq, f_s * nq), "mqa_fwd_kernel": (b_a * nq, f_a * nq),
                            "idx_select_kernel": (w.k * 4 * nq, 0), "idx_refine_kernel": (nv * 4 * nq, 0),
                            "mqa_combine_kernel": (2 * w.H * w.D * 2 * nq, 0)}
            self.calls = {"indexer_topk": (b_s * nq, f_s * nq), "sparse_mqa_fwd": (b_a * nq, f_a * nq)}
        else:
            b_a, f_a = _attention(w, nv + w.n_win, False)
            step_bytes = b_a * nq
            self.kernels = {"mqa_fwd_kernel": (b_a * nq, f_a * nq),
                            "mqa_combine_kernel": (2 * w.H * w.D * 2 * nq, 0)}
            self.calls = {"dense_compressed_mqa_fwd": (b_a * nq, f_a * nq)}
        self.bound = "hbm"
        self.launches = {}
        self.n_tokens = nq
        self.unit = "query-tokens/s"
        # enough copies of the caches that one step's data is evicted from the
        # Infinity Cache before the copy is used again
        self.copies = max(1, math.ceil(3 * CACHE_BYTES / step_bytes))
        # the resident cache and window rows hold prepared keys (kv_prepare runs
        # once per entry or token, when it is written; not part of a decode step)
        self.kv = [cakv.kv_prepare(inp["kv"].to(dev), m=w.m, rope_dims=w.rope_dims, rope_base=w.rope_base)
                   for _ in range(self.copies)]
        if self.sparse:
            self.kidx = [codes] + [codes.clone() for _ in range(self.copies - 1)]
            self.kscale = [scale] + [scale.clone() for _ in range(self.copies - 1)]
            self.q_idx = inp["q_idx"].to(dev)
            self.wts = inp["w"].to(dev)
            self.idx = torch.empty((w.B, w.Q, w.k), dtype=torch.int32, device=dev)
            self.ws_idx = torch.empty(cakv.indexer_topk_workspace_bytes(w.B, w.Q, w.N, w.k), dtype=torch.uint8,
                                      device=dev)
            ws_bytes = cakv.sparse_mqa_workspace_bytes(w.B, w.Q, w.H, w.D, w.k, w.n_win)
        else:
            ws_bytes = cakv.dense_mqa_workspace_bytes(w.B, w.Q, w.H, w.D, w.N, w.n_win)
        self.ws_attn = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        self.q = inp["q"].to(dev)
        self.kv_raw = cakv.kv_prepare_raw(inp["kv_raw"].to(dev), inp["raw_pos0"].tolist(), rope_dims=w.rope_dims,
                                          rope_base=w.rope_base)
        self.raw_pos0 = inp["raw_pos0"].to(dev)
        self.q_pos = inp["q_pos"].to(dev)
        self.sinks = inp["sinks"].to(dev)
        self.out = torch.empty((w.B, w.Q, w.H, w.D), dtype=torch.bfloat16, device=dev)
        self.kw = dict(m=w.m, n_win=w.n_win, rope_dims=w.rope_dims, rope_base=w.rope_base)
        self.inp = inp

    # ------------------------------------------------------------ prefill
    def _init_prefill(self, name):
        inp = make_inputs(name)
        w = self.w = inp["workload"]
        dev = "cuda"
        self.sparse = True
        self.copies = 1  # a step's working set (q, outputs) is several GB
        P, T, Q = w.q_pos0, w.T, w.Q
        assert P % w.m_hca == 0 and T % w.m_hca == 0 and w.B == 1
        self.P = P
        self.kv_raw = inp["kv_raw"].to(dev)  # the raw KV of prefix + chunk (window source)
        self.gate = inp["gate"].to(dev)
        self.hca_gate = inp["hca_gate"].to(dev)
        self.k_raw = inp["k_idx"].to(dev)
        self.k_gate = inp["k_gate"].to(dev)
        # prefix caches, built once outside the timed region (the chunk's part
        # is rewritten by every step)
        self.kvc = cakv.kv_compress(self.kv_raw, self.gate, w.m)
        self.kvh = cakv.kv_compress(self.kv_raw, self.hca_gate, w.m_hca)
        self.prep = dict(rope_dims=w.rope_dims, rope_base=w.rope_base)
        cakv.kv_prepare(self.kvc, m=w.m, **self.prep)
        cakv.kv_prepare(self.kvh, m=w.m_hca, **self.prep)
        # window rows: the raw tokens prepared at their positions (raw_pos0 = 0)
        self.kv_win = torch.empty_like(self.kv_raw)
        cakv.kv_prepare(self.kv_raw, m=1, j0=0, n=P, out=self.kv_win, **self.prep)
        self.codes, self.kscale = cakv.kv_compress(self.k_raw, self.k_gate, w.m, out_dtype=torch.float8_e4m3fn)
        self.q = inp["q"].to(dev)
        self.q_hca = inp["q_hca"].to(dev)
        self.q_idx = inp["q_idx"].to(dev)
        self.wts = inp["w"].to(dev)
        self.q_pos = inp["q_pos"].to(dev)
        self.raw_pos0 = inp["raw_pos0"].to(dev)
        self.sinks = inp["sinks"].to(dev)
        self.sinks_hca = inp["sinks_hca"].to(dev)
        N, Nh = T // w.m, T // w.m_hca
        self.idx = torch.empty((1, Q, w.k), dtype=torch.int32, device=dev)
        self.ws_idx = torch.empty(cakv.indexer_topk_workspace_bytes(1, Q, N, w.k), dtype=torch.uint8, device=dev)
        self.ws_csa = torch.empty(cakv.sparse_mqa_workspace_bytes(1, Q, w.H, w.D, w.k, w.n_win), dtype=torch.uint8,
                                  device=dev)
        self.ws_hca = torch.empty(cakv.dense_mqa_workspace_bytes(1, Q, w.H, w.D, Nh, w.n_win), dtype=torch.uint8,
                                  device=dev)
        self.out = torch.empty((1, Q, w.H, w.D), dtype=torch.bfloat16, device=dev)
        self.out_hca = torch.empty_like(self.out)
        self.kw = dict(n_win=w.n_win, rope_dims=w.rope_dims, rope_base=w.rope_base)
        self.inp = inp
        # algorithmic work of the whole chunk, summed over its query positions
        qs = P + np.arange(Q)
        nv_c, nv_h = qs // w.m, qs // w.m_hca
        win = np.minimum(qs + 1, w.n_win)
        f_score = int(np.sum(2 * w.HI * w.dI * nv_c))
        b_score = N * (w.dI + 4) + Q * (w.HI * w.dI * 2 + w.HI * 4)  # unique bytes: keys, scales, q_I, w
        rows_c = np.minimum(nv_c, w.k) + win
        rows_h = nv_h + win
        f_csa = int(np.sum(4 * w.H * w.D * rows_c))
        f_hca = int(np.sum(4 * w.H * w.D * rows_h))
        b_attn = (N + T) * w.D * 2 + 2 * Q * w.H * w.D * 2  # unique: caches, raw KV, q, out
        self.kernels = {"idx_score_fp8_kernel": (b_score, f_score), "mqa_fwd_kernel#0": (b_attn, f_csa),
                        "mqa_fwd_kernel#1": ((Nh + T) * w.D * 2 + 2 * Q * w.H * w.D * 2, f_hca)}
        self.calls = {"kv_compress x3, kv_prepare x3": (0, 0), "indexer_topk": (b_score, f_score),
                      "sparse_mqa_fwd": (b_attn, f_csa), "dense_compressed_mqa_fwd": (0, f_hca)}
        self.bound = "mfma"
        self.launches = {"mqa_fwd_kernel": 2}
        self.n_tokens = Q
        self.unit = "query-tokens/s"

    # ------------------------------------------------------------ one step
    def run(self, ev=None):
        (self._run_prefill if self.prefill else self._run_decode)(ev)

    def _run_decode(self, ev):
        c = self.i % self.copies
        self.i += 1
        if ev is not None:
            ev[0].record()
        if self.sparse:
            cakv.indexer_topk(self.q_idx, self.wts, self.kidx[c], self.kscale[c], self.q_pos, self.w.m, self.w.k,
                              out=self.idx, workspace=self.ws_idx)
            if ev is not None:
                ev[1].record()
            cakv.sparse_mqa_fwd(self.q, self.kv[c], self.idx, self.kv_raw, self.raw_pos0, self.q_pos, self.sinks,
                                want_lse=False, out=self.out, workspace=self.ws_attn, **self.kw)
            if ev is not None:
                ev[2].record()
        else:
            cakv.dense_compressed_mqa_fwd(self.q, self.kv[c], self.kv_raw, self.raw_pos0, self.q_pos, self.sinks,
                                          want_lse=False, out=self.out, workspace=self.ws_attn, **self.kw)
            if ev is not None:
                ev[1].record()

    def _run_prefill(self, ev):
        w, P = self.w, self.P
        if ev is not None:
            ev[0].record()
        cakv.kv_compress(self.kv_raw[:, P:], self.gate[:, P:], w.m, out=self.kvc[:, P // w.m:])
        cakv.kv_compress(self.kv_raw[:, P:], self.hca_gate[:, P:], w.m_hca, out=self.kvh[:, P // w.m_hca:])
        cakv.kv_compress(self.k_raw[:, P:], self.k_gate[:, P:], w.m, out=self.codes[:, P // w.m:],
                         scale=self.kscale[:, P // w.m:])
        # the chunk's new attention entries and its tokens' window rows enter prepared
        cakv.kv_prepare(self.kvc, m=w.m, j0=P // w.m, **self.prep)
        cakv.kv_prepare(self.kvh, m=w.m_hca, j0=P // w.m_hca, **self.prep)
        cakv.kv_prepare(self.kv_raw, m=1, j0=P, out=self.kv_win, **self.prep)
        if ev is not None:
            ev[1].record()
        cakv.indexer_topk(self.q_idx, self.wts, self.codes, self.kscale, self.q_pos, w.m, w.k, out=self.idx,
                          workspace=self.ws_idx)
        if ev is not None:
            ev[2].record()
        cakv.sparse_mqa_fwd(self.q, self.kvc, self.idx, self.kv_win, self.raw_pos0, self.q_pos, self.sinks, m=w.m,
                            want_lse=False, out=self.out, workspace=self.ws_csa, **self.kw)
        if ev is not None:
            ev[3].record()
        cakv.dense_compressed_mqa_fwd(self.q_hca, self.kvh, self.kv_win, self.raw_pos0, self.q_pos, self.sinks_hca,
                                      m=w.m_hca, want_lse=False, out=self.out_hca, workspace=self.ws_hca, **self.kw)
        if ev is not None:
            ev[4].record()

    @property
    def n_events(self) -> int:
        return len(self.calls) + 1

    def call_ms(self, evs):
        """Mean duration of each call of the step over the event-timed steps."""
        return {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(self.calls)}

    # ------------------------------------------------------------ oracle
    def cpu_baseline(self, max_queries: int, min_seconds: float):
        """The oracle on a bounded sample of the same inputs (all host cores),
        repeated until at least min_seconds of host time have passed."""
        import oracle
        self.cpu_seconds = min_seconds
        w, inp = self.w, self.inp
        if self.prefill:
            return self._cpu_baseline_prefill(oracle, max_queries)
        n = min(max_queries, w.B * w.Q)
        rows = np.arange(n, dtype=np.int64)
        if self.sparse:  # input preparation, outside the timed region
            codes, scale = oracle.q8_quantize(inp["k_idx"].numpy())
        kw = dict(m=w.m, n_win=w.n_win, rope_dims=w.rope_dims, rope_base=w.rope_base)

        def one_pass():
            if self.sparse:
                idx = oracle.indexer_topk(inp["q_idx"], inp["w"], inp["q_pos"], w.m, w.k, k_code=codes,
                                          k_scale=scale, rows=rows)
                full = np.full((w.B * w.Q, w.k), -1, np.int32)
                full[:n] = idx
                oracle.attention(inp["q"], inp["kv"], inp["kv_raw"], inp["raw_pos0"], inp["q_pos"], inp["sinks"],
                                 idx=full.reshape(w.B, w.Q, w.k), rows=rows, **kw)
            else:
                oracle.attention(inp["q"], inp["kv"], inp["kv_raw"], inp["raw_pos0"], inp["q_pos"], inp["sinks"],
                                 rows=rows, **kw)

        passes, dt = _repeat_for(one_pass, self.cpu_seconds)
        what = "oracle indexer + attention" if self.sparse else "oracle attention"
        return {"value": n * passes / dt, "unit": "query-tokens/s", "cores": _cores(), "kind": "oracle",
                "sample": f"{n} of the {w.B * w.Q} queries of {w.name} ({what}), {passes} passes",
                "seconds": round(dt, 3)}

    def _cpu_baseline_prefill(self, oracle, max_queries: int):
        """The oracle's chunk compressions in full, then indexer + both
        attention layers for the first n query tokens of the chunk."""
        w, inp, P = self.w, self.inp, self.P
        n = min(max_queries, w.Q)
        sl = slice(0, n)
        kv_chunk, kr_chunk = inp["kv"][:, P:], inp["k_idx"][:, P:]
        # prefix caches: input preparation, outside the timed region
        kvc_pre = oracle.kv_compress(inp["kv"][:, :P], inp["gate"][:, :P], w.m)
        kvh_pre = oracle.kv_compress(inp["kv"][:, :P], inp["hca_gate"][:, :P], w.m_hca)
        keys_pre = oracle.kv_compress(inp["k_idx"][:, :P], inp["k_gate"][:, :P], w.m)

        def one_pass():
            kvc = np.concatenate([kvc_pre, oracle.kv_compress(kv_chunk, inp["gate"][:, P:], w.m)], axis=1)
            kvh = np.concatenate([kvh_pre, oracle.kv_compress(kv_chunk, inp["hca_gate"][:, P:], w.m_hca)], axis=1)
            keys = np.concatenate([keys_pre, oracle.kv_compress(kr_chunk, inp["k_gate"][:, P:], w.m)], axis=1)
            codes, scale = oracle.q8_quantize(keys)
            idx = oracle.indexer_topk(inp["q_idx"][:, sl], inp["w"][:, sl], inp["q_pos"][:, sl], w.m, w.k,
                                      k_code=codes, k_scale=scale).reshape(1, n, w.k)
            kvc_t = torch.from_numpy(kvc).to(torch.bfloat16)
            kvh_t = torch.from_numpy(kvh).to(torch.bfloat16)
            oracle.attention(inp["q"][:, sl], kvc_t, inp["kv_raw"], inp["raw_pos0"], inp["q_pos"][:, sl],
                             inp["sinks"], idx=idx, m=w.m, **self.kw)
            oracle.attention(inp["q_hca"][:, sl], kvh_t, inp["kv_raw"], inp["raw_pos0"], inp["q_pos"][:, sl],
                             inp["sinks_hca"], m=w.m_hca, **self.kw)

        passes, dt = _repeat_for(one_pass, self.cpu_seconds)
        return {"value": n * passes / dt, "unit": "query-tokens/s", "cores": _cores(), "kind": "oracle",
                "sample": f"the chunk's three compressions, then indexer + CSA and HCA attention for the first {n} "
                          f"of the {w.Q} query tokens of {w.name}, {passes} passes",
                "seconds": round(dt, 3)}


class StreamStep:
    """The streaming decode step of a CSA layer and an HCA layer for 32
    sequences at 128K context (NEXT to the whole-batch calls: one new token
    per sequence per step).  Per step: one kv_append_batch of three appends
    (the token's KV into the CSA cache and window ring, its indexer key into
    the fp8 key cache, its KV into the HCA cache and window ring; a block
    completes every 4 tokens for CSA, every 128 for HCA), then indexer_topk,
    sparse_mqa_fwd and dense_compressed_mqa_fwd reading the window rings.  The prefix (131,072
    tokens: 32,768 CSA entries, 1,024 HCA entries) is built at set-up.  Three
    independent copies of the state are cycled (each advances one position
    every third step), so a step's caches are not Infinity-Cache resident."""

    name = "stream_decode_128k"
    prefill = False
    bound = "hbm"

    def __init__(self, copies: int = 3):
        inp = make_inputs("csa_decode_128k")
        w = self.w = inp["workload"]
        dev = "cuda"
        B, D, m, mh, t0 = w.B, w.D, w.m, w.m_hca, w.t
        self.copies = copies
        self.t = [t0] * copies
        self.max_steps = 1 << 14
        N = t0 // m + self.max_steps // m + 2
        Nh = t0 // mh + self.max_steps // mh + 2
        g = torch.Generator(device="cpu").manual_seed(11)
        prep = self.prep = dict(rope_dims=w.rope_dims, rope_base=w.rope_base, entry_pos_offset=0, rms_eps=w.rms_eps)
        self.state = []
        kf = inp["k_idx"].to(dev)
        codes, scale = cakv.kv_compress(kf, torch.zeros(kf.shape[:2], dtype=torch.float32, device=dev), 1,
                                        out_dtype=torch.float8_e4m3fn)
        del kf
        hca_prefix = torch.randn(B, t0 // mh, D, generator=g).to(torch.bfloat16)
        for c in range(copies):
            st = {}
            st["kv"] = torch.zeros(B, N, D, dtype=torch.bfloat16, device=dev)
            st["kv"][:, : t0 // m] = inp["kv"].to(dev)
            cakv.kv_prepare(st["kv"], m=m, n=t0 // m, **prep)
            st["kh"] = torch.zeros(B, Nh, D, dtype=torch.bfloat16, device=dev)
            st["kh"][:, : t0 // mh] = hca_prefix.to(dev)
            cakv.kv_prepare(st["kh"], m=mh, n=t0 // mh, **prep)
            st["kc"] = torch.zeros(B, N, w.dI, dtype=torch.uint8, device=dev).view(torch.float8_e4m3fn)
            st["ks"] = torch.zeros(B, N, dtype=torch.float32, device=dev)
            st["kc"][:, : t0 // m] = codes
            st["ks"][:, : t0 // m] = scale
            # rings: raw tokens and gates of the last 128 positions, window rows prepared at them
            raw = torch.randn(B, 128, D, generator=g).to(torch.bfloat16).to(dev)
            st["raw_c"], st["raw_h"] = raw.clone(), raw.clone()
            st["graw_c"] = torch.randn(B, 128, generator=g).to(dev)
            st["graw_h"] = torch.randn(B, 128, generator=g).to(dev)
            st["kraw"] = torch.randn(B, 8, w.dI, generator=g).to(torch.bfloat16).to(dev)
            st["kgraw"] = torch.randn(B, 8, generator=g).to(dev)
            win = torch.empty_like(raw)
            p = torch.arange(t0 - 128, t0, device=dev)
            win[:, p % 128] = cakv.kv_prepare(raw[:, p % 128].contiguous(), m=1, entry_pos_offset=t0 - 128,
                                              rope_dims=w.rope_dims, rope_base=w.rope_base)
            st["win_c"], st["win_h"] = win.clone(), win.clone()
            self.state.append(st)
        # the new tokens: a pool cycled over the steps
        P = 64
        self.tok = torch.randn(P, B, D, generator=g).to(torch.bfloat16).to(dev)
        self.ktok = torch.randn(P, B, w.dI, generator=g).to(torch.bfloat16).to(dev)
        self.gtok = torch.randn(P, 3, B, generator=g).to(dev)
        self.q = inp["q"].to(dev)
        self.qh = inp["q"].to(dev).flip(2).contiguous()  # the HCA layer's query heads
        self.q_idx = inp["q_idx"].to(dev)
        self.wts = inp["w"].to(dev)
        self.sinks = inp["sinks"].to(dev)
        self.idx = torch.empty((B, 1, w.k), dtype=torch.int32, device=dev)
        self.ws_idx = torch.empty(cakv.indexer_topk_workspace_bytes(B, 1, N, w.k), dtype=torch.uint8, device=dev)
        self.ws_a = torch.empty(max(cakv.sparse_mqa_workspace_bytes(B, 1, w.H, D, w.k, w.n_win), 1),
                                dtype=torch.uint8, device=dev)
        self.ws_h = torch.empty(max(cakv.dense_mqa_workspace_bytes(B, 1, w.H, D, Nh, w.n_win), 1),
                                dtype=torch.uint8, device=dev)
        self.out = torch.empty((B, 1, w.H, D), dtype=torch.bfloat16, device=dev)
        self.out_h = torch.empty_like(self.out)
        # positions of every step, one row per step (no fill kernel inside a step)
        self.pos_table = (t0 + torch.arange(self.max_steps, dtype=torch.int32, device=dev))[:, None].repeat(1, B)
        self.P = P
        self.i = 0
        nv, nvh = t0 // m, t0 // mh
        b_s, f_s = _indexer_score(w, nv)
        b_a, f_a = _attention(w, w.k + w.n_win, True)
        b_h, f_h = _attention(w, nvh + w.n_win, False)
        b_app = 3 * D * 2 + 2 * D * 2 + w.dI * 2 + 3 * 4  # token rows in, ring and window rows out
        self.kernels = {"idx_score_fp8_kernel": (b_s * B, f_s * B), "mqa_fwd_kernel#0": (b_a * B, f_a * B),
                        "mqa_fwd_kernel#1": (b_h * B, f_h * B), "kv_append_kernel#0": (b_app * B, 0)}
        self.launches = {"mqa_fwd_kernel": 2, "kv_append_kernel": 1}
        self.calls = {"kv_append_batch (3 appends)": (b_app * B, 0), "indexer_topk": (b_s * B, f_s * B),
                      "sparse_mqa_fwd (ring window)": (b_a * B, f_a * B),
                      "dense_compressed_mqa_fwd (ring window)": (b_h * B, f_h * B)}
        self.n_tokens = B
        self.unit = "query-tokens/s"
        self.config = {"workload": self.name, "batch": B, "context": t0, "m": m, "m_hca": mh, "heads": w.H,
                       "head_dim": D, "topk": w.k, "window": w.n_win, "state_copies_cycled": copies,
                       "step": "kv_append_batch (3 appends) + indexer_topk + sparse_mqa_fwd + dense_compressed_mqa_fwd"}

    @property
    def n_events(self) -> int:
        return len(self.calls) + 1

    def call_ms(self, evs):
        return {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(self.calls)}

    def run(self, ev=None):
        c = self.i % self.copies
        j = (self.i // self.copies) % self.P
        self.i += 1
        st, w = self.state[c], self.w
        if self.t[c] - w.t >= self.max_steps - 1:  # stay inside the allocated caches
            self.t[c] = w.t
        pos = self.pos_table[self.t[c] - w.t]
        self.t[c] += 1
        kw = dict(n_win=w.n_win, rope_dims=w.rope_dims, rope_base=w.rope_base)
        if ev is not None:
            ev[0].record()
        tok = self.tok[j]
        cakv.kv_append_batch([
            dict(x_tok=tok, gate_tok=self.gtok[j, 0], raw_ring=st["raw_c"], gate_ring=st["graw_c"], cache=st["kv"],
                 m=w.m, win_ring=st["win_c"], prep=self.prep),
            dict(x_tok=self.ktok[j], gate_tok=self.gtok[j, 1], raw_ring=st["kraw"], gate_ring=st["kgraw"],
                 cache=st["kc"], m=w.m, cache_scale=st["ks"]),
            dict(x_tok=tok, gate_tok=self.gtok[j, 2], raw_ring=st["raw_h"], gate_ring=st["graw_h"], cache=st["kh"],
                 m=w.m_hca, win_ring=st["win_h"], prep=self.prep)], pos)
        if ev is not None:
            ev[1].record()
        qpos = pos.view(-1, 1)
        cakv.indexer_topk(self.q_idx, self.wts, st["kc"], st["ks"], qpos, w.m, w.k, out=self.idx,
                          workspace=self.ws_idx)
        if ev is not None:
            ev[2].record()
        cakv.sparse_mqa_fwd(self.q, st["kv"], self.idx, st["win_c"], None, qpos, self.sinks, m=w.m, raw_ring=True,
                            want_lse=False, out=self.out, workspace=self.ws_a, **kw)
        if ev is not None:
            ev[3].record()
        cakv.dense_compressed_mqa_fwd(self.qh, st["kh"], st["win_h"], None, qpos, self.sinks, m=w.m_hca,
                                      raw_ring=True, want_lse=False, out=self.out_h, workspace=self.ws_h, **kw)
        if ev is not None:
            ev[4].record()


class CompressStep:
    """The compressor variants on a 262,144-token prefix: overlapping spans of
    8 tokens at m = 4 with one gate logit per token and channel (bf16 KV
    [1, 262144, 512], float32 gates [1, 262144, 512] ~N(0,1), seed 7), bf16
    entries.  One step = one kv_compress_ex call (65,536 entries)."""

    name = "compress_variants_256k"
    prefill = False
    bound = "hbm"

    def __init__(self):
        dev = "cuda"
        T, D, self.m, self.span = 262144, 512, 4, 8
        rng = np.random.Generator(np.random.PCG64(7))
        self.x = torch.from_numpy(rng.standard_normal((1, T, D), dtype=np.float32)).to(torch.bfloat16).to(dev)
        self.g = torch.from_numpy(rng.standard_normal((1, T, D), dtype=np.float32)).to(dev)
        self.out = torch.empty((1, T // self.m, D), dtype=torch.bfloat16, device=dev)
        b = T * D * 2 + T * D * 4 + (T // self.m) * D * 2  # tokens, gates, entries, each once
        self.kernels = {"kv_compress_kernel": (b, 0)}
        self.launches = {"kv_compress_kernel": 1}
        # both compressor kernels share the launch marker; at m = 4, span 8 the run kernel runs
        self.profile_names = {"kv_compress_kernel": "kv_compress_run_kernel"}
        self.calls = {"kv_compress_ex": (b, 0)}
        self.copies = 1
        self.n_tokens = T
        self.unit = "tokens/s"
        self.config = {"workload": self.name, "tokens": T, "head_dim": D, "m": self.m, "span": self.span,
                       "gates": "per token and channel", "out": "bf16"}

    @property
    def n_events(self) -> int:
        return 2

    def call_ms(self, evs):
        return {"kv_compress_ex": float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))}

    def run(self, ev=None):
        if ev is not None:
            ev[0].record()
        cakv.kv_compress_ex(self.x, self.g, self.m, self.span, out=self.out)
        if ev is not None:
            ev[1].record()


class BackwardStep:
    """The training backward of a CSA layer at the 128K decode shapes (32
    queries, 128 heads x 512, 1,024 selected entries + a 128-token window,
    64 indexer heads x 128 over the selection): mqa_bwd (dq, the prepared
    key rows' and the sinks' gradients) and indexer_bwd.  Forward output, lse
    and selection come from one forward pass at set-up; dout and dS are
    ~N(0,1).  The gradient buffers accumulate across steps (as a gradient
    accumulation would)."""

    name = "backward_csa_decode_128k"
    prefill = False
    bound = "mfma"

    def __init__(self):
        inp = make_inputs("csa_decode_128k")
        w = self.w = inp["workload"]
        dev = "cuda"
        B, Q, H, D = w.B, w.Q, w.H, w.D
        kf = inp["k_idx"].to(dev)
        self.codes, self.kscale = cakv.kv_compress(kf, torch.zeros(kf.shape[:2], dtype=torch.float32, device=dev),
                                                   1, out_dtype=torch.float8_e4m3fn)
        del kf
        self.kv = cakv.kv_prepare(inp["kv"].to(dev), m=w.m, rope_dims=w.rope_dims, rope_base=w.rope_base)
        self.kv_raw = cakv.kv_prepare_raw(inp["kv_raw"].to(dev), inp["raw_pos0"].tolist(), rope_dims=w.rope_dims,
                                          rope_base=w.rope_base)
        self.q, self.q_idx, self.wts = inp["q"].to(dev), inp["q_idx"].to(dev), inp["w"].to(dev)
        self.raw_pos0, self.q_pos, self.sinks = inp["raw_pos0"].to(dev), inp["q_pos"].to(dev), inp["sinks"].to(dev)
        self.kw = dict(m=w.m, n_win=w.n_win, rope_dims=w.rope_dims, rope_base=w.rope_base)
        self.idx = cakv.indexer_topk(self.q_idx, self.wts, self.codes, self.kscale, self.q_pos, w.m, w.k)
        self.out, self.lse = cakv.sparse_mqa_fwd(self.q, self.kv, self.idx, self.kv_raw, self.raw_pos0, self.q_pos,
                                                 self.sinks, **self.kw)
        g = torch.Generator(device="cpu").manual_seed(13)
        self.dout = torch.randn(B, Q, H, D, generator=g).to(dev)
        self.dS = torch.randn(B, Q, w.k, generator=g).to(dev)
        self.dkv = torch.zeros(B, w.N, D, dtype=torch.float32, device=dev)
        self.draw = torch.zeros(B, w.n_win, D, dtype=torch.float32, device=dev)
        self.dsinks = torch.zeros(H, dtype=torch.float32, device=dev)
        self.dk = torch.zeros(B, w.N, w.dI, dtype=torch.float32, device=dev)
        self.ws = torch.empty(cakv.load_library().cakv_mqa_bwd_workspace(B, Q, H, D, w.k, w.n_win),
                              dtype=torch.uint8, device=dev)
        nq, rows = B * Q, w.k + w.n_win
        # algorithmic work: attention 10 H D flops per key (S, dP, dq, and the two dK products), the key rows
        # read and their gradients written once, q / out / dout / dq; indexer 6 HI dI flops per selected entry
        f_att = 10 * H * D * rows * nq
        b_att = (rows * D * 2 + rows * D * 4 + 4 * H * D * 4) * nq
        f_idx = 6 * w.HI * w.dI * w.k * nq
        b_idx = (w.k * (w.dI + 4) + w.k * w.dI * 4 + w.k * 8 + 2 * w.HI * w.dI * 4) * nq
        self.kernels = {"bwd_logits_kernel": (0, 4 * H * D * rows * nq), "bwd_dkeys_kernel": (0, 4 * H * D * rows * nq),
                        "bwd_dquery_kernel": (0, 2 * H * D * rows * nq), "indexer_bwd_kernel": (b_idx, f_idx)}
        self.kernel_bound = {"indexer_bwd_kernel": "alu"}  # fp32 VALU (the canonical-order score)
        self.launches = {}
        self.calls = {"mqa_bwd": (b_att, f_att), "indexer_bwd": (b_idx, f_idx)}
        self.copies = 1
        self.n_tokens = nq
        self.unit = "query-tokens/s"
        self.config = {"workload": self.name, "batch": nq, "context": w.t, "heads": H, "head_dim": D, "topk": w.k,
                       "window": w.n_win, "indexer_heads": w.HI, "step": "mqa_bwd + indexer_bwd"}

    @property
    def n_events(self) -> int:
        return 3

    def call_ms(self, evs):
        return {n: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) for i, n in enumerate(self.calls)}

    def run(self, ev=None):
        if ev is not None:
            ev[0].record()
        cakv.mqa_bwd(self.q, self.kv, self.idx, self.kv_raw, self.raw_pos0, self.q_pos, self.sinks, self.out,
                     self.lse, self.dout, dkv_c=self.dkv, dkv_raw=self.draw, dsinks=self.dsinks, workspace=self.ws,
                     **self.kw)
        if ev is not None:
            ev[1].record()
        cakv.indexer_bwd(self.q_idx, self.wts, self.codes, self.kscale, self.q_pos, self.idx, self.dS, self.w.m,
                         dk=self.dk)
        if ev is not None:
            ev[2].record()


def _repeat_for(fn, min_seconds: float):
    """Runs fn until at least min_seconds have passed (at least once);
    returns (passes, seconds)."""
    passes, t0 = 0, time.perf_counter()
    while True:
        fn()
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            return passes, dt


def _cores() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))


def copy_calibration(mib: int):
    """A plain copy kernel of known size: each launch reads and writes exactly
    `mib` MiB, the yardstick for the FETCH_SIZE / WRITE_SIZE counters."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n, "launches": 5}), flush=True)


def _kernel_launches(st, kernel: str):
    """(name, occurrence, launches per step) of a kernel table entry:
    'mqa_fwd_kernel#1' is the second launch of mqa_fwd_kernel in a step."""
    name, _, occ = kernel.partition("#")
    return name, int(occ or 0), getattr(st, "launches", {}).get(name, 1)


def _time_kernel(st: Step, kernel: str, steps: int, run_steps):
    """Mean duration (ms) of one kernel's launches over `steps` steps, from
    event pairs the library records around them."""
    name, occ, per_step = _kernel_launches(st, kernel)
    n = steps * per_step
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    cakv.profile_kernel_events(name, starts, ends)
    run_steps()
    torch.cuda.synchronize()
    cakv.profile_kernel_events(None)
    return float(np.mean([starts[i].elapsed_time(ends[i]) for i in range(occ, n, per_step)]))


def _event_pair_ms(n: int = 50) -> float:
    """Median interval of an empty HIP event pair on the current stream: the
    markers' own latency, subtracted from the event-timed kernel durations."""
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for a, b in pairs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in pairs]))


def _source_digest() -> str:
    """sha256 of libcakv.so's sources (its kernels and the headers), sorted
    by name; the measurement probes are built apart and left out."""
    import hashlib
    from compressed_attention_kv_amd.build import SOURCES
    h = hashlib.sha256()
    cs = os.path.join(ROOT, "compressed_attention_kv_amd", "csrc")
    for f in sorted(os.listdir(cs)):
        if f.endswith(".hpp") or f in SOURCES:
            h.update(f.encode())
            h.update(open(os.path.join(cs, f), "rb").read())
    return h.hexdigest()


def _profiled(workload: str, kernel: str, key: str):
    """A figure of `kernel` from the committed summary of this workload
    (profiles/<workload>_kernels.md): the line '<key>: kernel=... value=...
    source_sha256=...' taken while the library sources hashed to the same
    digest as now, else None."""
    f = os.path.join(ROOT, "profiles", f"{workload}_kernels.md")
    if not os.path.exists(f):
        return None
    digest = _source_digest()
    for line in open(f):
        if line.startswith(key + ":"):
            kv = dict(t.split("=", 1) for t in line.split()[1:] if "=" in t)
            if kv.get("kernel") == kernel and kv.get("source_sha256") == digest:
                return float(kv["value"])
    return None


PEAKS = {"hbm": (HBM_PEAK_GBS, "GB/s"), "mfma": (BF16_PEAK_TFS, "TFLOP/s"), "alu": (FP32_VALU_PEAK_TFS, "TFLOP/s")}
# what this GPU reaches, measured by attainable_peaks() before the workloads
# (empty: the fractions against it are left out)
ATTAINABLE = {}
_ATT_KEY = {"hbm": "hbm_read_GBps", "mfma": "bf16_mfma_TFLOPs"}


def attainable_peaks(read_gib: int = 4, mfma_iters: int = 32768, mfma_blocks: int = 512) -> dict:
    """The GPU's attainable peaks from libcakv_probes.so: a streaming read of
    a read_gib GiB buffer (2,048 workgroups on contiguous ranges, nontemporal
    16-byte loads, eight in flight per thread; median of five after one
    untimed read) and the bf16 MFMA loop
    (mfma_blocks workgroups of four waves, two per SIMD, each running four
    independent 32x32x16 chains; median of three after one untimed launch)."""
    def timed(fn, n):
        ts = []
        for _ in range(n):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            b.synchronize()
            ts.append(a.elapsed_time(b))
        return float(np.median(ts))
    nbytes = read_gib << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")  # (written once: no first-touch cost)
    sink = torch.empty(2048, dtype=torch.int32, device="cuda")
    cakv.probe_read(buf, sink)
    t_read = timed(lambda: cakv.probe_read(buf, sink), 5)
    del buf
    msink = torch.empty(4 * mfma_blocks, dtype=torch.float32, device="cuda")
    flops = cakv.probe_mfma_bf16(mfma_iters, mfma_blocks, msink)
    t_mfma = timed(lambda: cakv.probe_mfma_bf16(mfma_iters, mfma_blocks, msink), 3)
    torch.cuda.empty_cache()
    return {"hbm_read_GBps": round(nbytes / (t_read * 1e-3) / 1e9, 1), "read_bytes": nbytes,
            "read_ms": round(t_read, 4), "bf16_mfma_TFLOPs": round(flops / (t_mfma * 1e-3) / 1e12, 1),
            "mfma_flops": flops, "mfma_ms": round(t_mfma, 4),
            "probes": "libcakv_probes.so (include/cakv_probes.h): streaming read, bf16 MFMA loop"}


def measure(st, steps: int, warmup: int) -> dict:
    """Times `steps` steps of a workload (three windows, the median one
    reported) and the roofline of its dominant kernel."""
    for _ in range(warmup):
        st.run()
    torch.cuda.synchronize()
    pair_ms = _event_pair_ms()
    # the dominant kernel: the longest of the step's main kernels on a short
    # probe; kernels within 10 % of the longest count as a tie, which goes to
    # the one with the most algorithmic work (bytes when HBM-bound, flops
    # otherwise), so that timing noise cannot flip the choice
    probe = {k: _time_kernel(st, k, 4, lambda: [st.run() for _ in range(4)]) for k in st.kernels}
    top = max(probe.values())
    dom = max((k for k in probe if probe[k] >= 0.9 * top), key=lambda k: st.kernels[k][0 if st.bound == "hbm" else 1])
    dom_name, occ, per_step = _kernel_launches(st, dom)
    bound = getattr(st, "kernel_bound", {}).get(dom_name, st.bound)

    # per-call breakdown: an untimed pass with HIP events around each call
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(st.n_events)] for _ in range(steps)]
    for i in range(steps):
        st.run(evs[i])
    torch.cuda.synchronize()

    # timed region: `steps` steps; the only events in it are the ones the
    # library records around each launch of the dominant kernel.  Three such
    # windows run back to back and the median one is reported (all three are
    # listed): a host-side stall outside the kernels then cannot stand for
    # the path's throughput.
    windows = []
    for _ in range(3):
        ks = [torch.cuda.Event(enable_timing=True) for _ in range(steps * per_step)]
        ke = [torch.cuda.Event(enable_timing=True) for _ in range(steps * per_step)]
        cakv.profile_kernel_events(dom_name, ks, ke)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            st.run()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        cakv.profile_kernel_events(None)
        k_raw = float(np.mean([ks[i].elapsed_time(ke[i]) for i in range(occ, steps * per_step, per_step)]))
        windows.append((wall, k_raw))
    wall, kms_raw = sorted(windows)[1]
    kms = kms_raw - pair_ms
    ms = wall * 1e3 / steps
    value = st.n_tokens / (ms * 1e-3)

    bytes_, flops = st.kernels[dom]
    peak, unit = PEAKS[bound]
    work = bytes_ if bound == "hbm" else flops
    scale = 1e9 if bound == "hbm" else 1e12
    achieved = work / (kms * 1e-3) / scale
    # the kernel's name in the trace, where its launches' event marker is shared
    prof_name = getattr(st, "profile_names", {}).get(dom_name, dom_name)
    rp_us = _profiled(st.name, prof_name, "duration_us")
    roof = {"kernel": dom, "bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4),
            "traffic": (lambda v: None if v is None else int(v))(_profiled(st.name, prof_name, "traffic_bytes")),
            "kernel_ms": round(kms, 4), "kernel_ms_events_raw": round(kms_raw, 4), "event_pair_ms": round(pair_ms, 4),
            "frac_events_raw": round(work / (kms_raw * 1e-3) / scale / peak, 4), "launches_timed": steps}
    if rp_us:
        roof["kernel_ms_rocprof"] = round(rp_us * 1e-3, 4)
        roof["frac_rocprof"] = round(work / (rp_us * 1e-6) / scale / peak, 4)
    att = ATTAINABLE.get(_ATT_KEY.get(bound, ""))
    if att:
        roof["attainable_peak"] = att
        roof["frac_attainable"] = round(achieved / att, 4)
    cms = st.call_ms(evs)
    per_call = {}
    for c, (b, f) in st.calls.items():
        d = {"ms": round(cms[c], 4)}
        if b:
            d["alg_GBps"] = round(b / (cms[c] * 1e-3) / 1e9, 1)
            d["hbm_frac"] = round(b / (cms[c] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
        if f:
            d["alg_TFLOPs"] = round(f / (cms[c] * 1e-3) / 1e12, 1)
            d["mfma_frac_bf16"] = round(f / (cms[c] * 1e-3) / 1e12 / BF16_PEAK_TFS, 4)
        per_call[c] = d
    if st.bound == "hbm":
        roof_ms = sum(b for b, _ in st.calls.values()) / (HBM_PEAK_GBS * 1e9) * 1e3
    else:
        roof_ms = sum(f for _, f in st.calls.values()) / (BF16_PEAK_TFS * 1e12) * 1e3
    rec = {"value": round(value, 1), "unit": st.unit, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4),
           "config": st.config, "windows_ms_per_step": [round(wl * 1e3 / steps, 4) for wl, _ in windows],
           "roofline": roof, "path_roofline_frac": round(roof_ms / ms, 4), "path_bound": st.bound,
           "per_call": per_call, "kernel_probe_ms": {k: round(v, 4) for k, v in probe.items()}}
    path_att = ATTAINABLE.get(_ATT_KEY.get(st.bound, ""))
    if path_att:
        # the same roofline time priced at what this GPU reaches
        rec["path_roofline_frac_attainable"] = round(roof_ms * PEAKS[st.bound][0] / path_att / ms, 4)
    return rec


FORWARD = ["csa_decode_128k", "csa_decode_1m", "hca_decode_1m", "prefill_chunk_256k", "flash_csa_decode_128k",
           "flash_hca_decode_1m"]
EXTRA = {"stream_decode_128k": StreamStep, "compress_variants_256k": CompressStep,
         "backward_csa_decode_128k": BackwardStep}
HEADLINE = "csa_decode_128k"


def make_step(name: str):
    if name in EXTRA:
        return EXTRA[name]()
    st = Step(name)
    st.name = name
    w = st.w
    if st.prefill:
        st.config = {"workload": w.name, "query_tokens": w.Q, "prefix_tokens": w.q_pos0, "m": w.m, "m_hca": w.m_hca,
                     "heads": w.H, "head_dim": w.D, "topk": w.k, "window": w.n_win, "indexer_heads": w.HI,
                     "layers": "CSA + HCA"}
    else:
        st.config = {"workload": w.name, "batch": w.B * w.Q, "context": w.t, "compressed_entries": w.N, "m": w.m,
                     "heads": w.H, "head_dim": w.D, "topk": w.k if st.sparse else None, "window": w.n_win,
                     "indexer_heads": w.HI if st.sparse else None, "cache_copies_cycled": st.copies}
    return st


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default 50; 5 for the prefill chunk)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps (default 5; 2 for the prefill chunk)")
    ap.add_argument("--workload", default=HEADLINE, choices=FORWARD + list(EXTRA),
                    help="the workload of the line's top-level figures")
    ap.add_argument("--extras", default="all", choices=["all", "none"],
                    help="also measure every other workload (reported under 'workloads', no CPU baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-queries", type=int, default=32)
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="the oracle baseline repeats its sample until this much host time has passed")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (HBM counter calibration)")
    ap.add_argument("--no-attainable", action="store_true",
                    help="skip the attainable-peak probes (fractions against the published peaks only)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    torch.cuda.init()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    def counts(name):
        prefill = name.startswith("prefill")
        return (args.steps if args.steps is not None else (5 if prefill else 50),
                args.warmup if args.warmup is not None else (2 if prefill else 5))

    if not args.no_attainable:
        ATTAINABLE.update(attainable_peaks())
    steps, warmup = counts(args.workload)
    st = make_step(args.workload)
    rec = measure(st, steps, warmup)
    line = {"metric": METRIC, "value": rec.pop("value"), "unit": rec.pop("unit"), "n_gpus": 1,
            "steps": rec.pop("steps"), "warmup": rec.pop("warmup"), "ms_per_step": rec.pop("ms_per_step"),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "dtype_detail": "bf16 MFMA with fp32 accumulation (indexer: fp8 keys decoded exactly to bf16)",
            "data": "synthetic", "config": rec.pop("config")}
    line.update(rec)
    if ATTAINABLE:
        line["attainable"] = dict(ATTAINABLE)
    if not args.no_cpu_baseline and hasattr(st, "cpu_baseline"):
        q = args.cpu_queries if not st.prefill else min(args.cpu_queries, 8)
        line["cpu_baseline"] = st.cpu_baseline(q, args.cpu_seconds)
    del st
    torch.cuda.empty_cache()
    if args.extras == "all":
        line["workloads"] = {}
        for name in FORWARD + list(EXTRA):
            if name == args.workload:
                continue
            s2, w2 = counts(name)
            print(f"# measuring {name}", file=sys.stderr, flush=True)
            st = make_step(name)
            line["workloads"][name] = measure(st, s2, w2)
            del st
            torch.cuda.empty_cache()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
