"""Throughput of the compressed-attention hot path on one MI355X.

Default workload: CSA decode at 128K context -- 32 sequences, each query at
position 131072 over 32768 compressed entries (m=4) with fp8 indexer keys,
top-1024 selection, then sparse MQA (128 heads x 512) over the selection plus
the 128-token raw window and the sinks.  One step = indexer_topk +
sparse_mqa_fwd for the batch, inputs resident in HBM.  Other workloads
(--workload): csa_decode_1m, hca_decode_1m (dense_compressed_mqa_fwd only).

The timed region cycles through several copies of the caches so that the
256 MiB Infinity Cache cannot hold a step's working set between steps.

Prints one JSON line (metric, value, roofline of the dominant kernel call,
CPU-oracle baseline).  --gpus N with N > 1 is not supported: this build runs
on one GPU.
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
CACHE_BYTES = 256 << 20


def _alg_bytes_indexer(w) -> int:
    # per query: fp8 keys + per-entry scales of every visible entry, the
    # indexer query heads (bf16), head weights (f32), the k output indices
    nv = min(w.t // w.m, w.N)
    return nv * w.dI + nv * 4 + w.HI * w.dI * 2 + w.HI * 4 + w.k * 4


def _alg_bytes_attention(w, sparse: bool) -> int:
    nv = min(w.t // w.m, w.N)
    rows = (w.k if sparse else nv) + w.n_win
    return rows * w.D * 2 + w.H * w.D * 2 * 2 + (w.k * 4 if sparse else 0) + w.H * 4


def _alg_flops_attention(w, sparse: bool) -> int:
    nv = min(w.t // w.m, w.N)
    rows = (w.k if sparse else nv) + w.n_win
    return 4 * w.H * w.D * rows


def _alg_flops_indexer(w) -> int:
    nv = min(w.t // w.m, w.N)
    return 2 * w.HI * w.dI * nv


class Step:
    """Device-resident inputs (several copies of the caches) and one step of the path."""

    def __init__(self, name: str):
        self.name = name
        inp = make_inputs(name)
        w = self.w = inp["workload"]
        dev = "cuda"
        self.sparse = w.csa
        ws_bytes = 0
        nq = w.B * w.Q
        if self.sparse:
            # the indexer key cache in fp8 + per-entry scale: kv_compress with
            # m = 1 is exactly the per-entry quantiser
            kf = inp["k_idx"].to(dev)
            codes, scale = cakv.kv_compress(kf, torch.zeros(kf.shape[:2], dtype=torch.float32, device=dev), 1,
                                            out_dtype=torch.float8_e4m3fn)
            del kf
            step_bytes = (_alg_bytes_indexer(w) + _alg_bytes_attention(w, True)) * nq
        else:
            step_bytes = _alg_bytes_attention(w, False) * nq
        # enough copies of the caches that one step's data is evicted from the
        # Infinity Cache before the copy is used again
        self.copies = max(1, math.ceil(3 * CACHE_BYTES / step_bytes))
        self.kv = [inp["kv"].to(dev) for _ in range(self.copies)]
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
        self.kv_raw = inp["kv_raw"].to(dev)
        self.raw_pos0 = inp["raw_pos0"].to(dev)
        self.q_pos = inp["q_pos"].to(dev)
        self.sinks = inp["sinks"].to(dev)
        self.out = torch.empty((w.B, w.Q, w.H, w.D), dtype=torch.bfloat16, device=dev)
        self.kw = dict(m=w.m, n_win=w.n_win, rope_dims=w.rope_dims, rope_base=w.rope_base)
        self.inp = inp
        self.i = 0

    def run(self, ev=None):
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
        else:
            if ev is not None:
                ev[1].record()
            cakv.dense_compressed_mqa_fwd(self.q, self.kv[c], self.kv_raw, self.raw_pos0, self.q_pos, self.sinks,
                                          want_lse=False, out=self.out, workspace=self.ws_attn, **self.kw)
        if ev is not None:
            ev[2].record()

    def cpu_baseline(self, max_queries: int):
        """The oracle on the first `n` queries of the same inputs (all host cores)."""
        import oracle
        w, inp = self.w, self.inp
        n = min(max_queries, w.B * w.Q)
        rows = np.arange(n, dtype=np.int64)
        if self.sparse:  # input preparation, outside the timed region
            codes, scale = oracle.q8_quantize(inp["k_idx"].numpy())
        t0 = time.perf_counter()
        kw = dict(m=w.m, n_win=w.n_win, rope_dims=w.rope_dims, rope_base=w.rope_base)
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
        dt = time.perf_counter() - t0
        cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
        return {"value": n / dt, "unit": "query-tokens/s", "cores": cores, "kind": "oracle",
                "sample": f"{n} of the {w.B * w.Q} queries of {w.name} (oracle indexer + attention)"
                if self.sparse else f"{n} of the {w.B * w.Q} queries of {w.name} (oracle attention)",
                "seconds": round(dt, 3)}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="csa_decode_128k",
                    choices=["csa_decode_128k", "csa_decode_1m", "hca_decode_1m"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-queries", type=int, default=32)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    torch.cuda.init()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    st = Step(args.workload)
    w = st.w
    for _ in range(args.warmup):
        st.run()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        st.run(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    idx_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    att_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    ms = wall * 1e3 / args.steps
    nq = w.B * w.Q
    value = nq / (ms * 1e-3)

    # roofline of the dominant call (HBM-bound): algorithmic bytes / its event-timed duration
    if st.sparse:
        b_idx = _alg_bytes_indexer(w) * nq
        b_att = _alg_bytes_attention(w, True) * nq
        calls = {"indexer_topk": (b_idx, idx_ms, _alg_flops_indexer(w) * nq),
                 "sparse_mqa_fwd": (b_att, att_ms, _alg_flops_attention(w, True) * nq)}
    else:
        calls = {"dense_compressed_mqa_fwd": (_alg_bytes_attention(w, False) * nq, att_ms,
                                              _alg_flops_attention(w, False) * nq)}
    dom = max(calls, key=lambda c: calls[c][1])
    bytes_, dms, flops = calls[dom]
    achieved = bytes_ / (dms * 1e-3) / 1e9
    per_call = {c: {"ms": round(v[1], 4), "alg_GBps": round(v[0] / (v[1] * 1e-3) / 1e9, 1),
                    "hbm_frac": round(v[0] / (v[1] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "alg_TFLOPs": round(v[2] / (v[1] * 1e-3) / 1e12, 1),
                    "mfma_frac_bf16": round(v[2] / (v[1] * 1e-3) / 1e12 / BF16_PEAK_TFS, 4)}
                for c, v in calls.items()}
    total_bytes = sum(v[0] for v in calls.values())
    roof_ms = total_bytes / (HBM_PEAK_GBS * 1e9) * 1e3
    rec = {
        "metric": METRIC, "value": round(value, 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8 keys decoded to bf16 MFMA (indexer), f16 MFMA (attention), fp32 accumulate",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": nq, "context": w.t, "compressed_entries": w.N, "m": w.m,
                   "heads": w.H, "head_dim": w.D, "topk": w.k if st.sparse else None, "window": w.n_win,
                   "indexer_heads": w.HI if st.sparse else None, "cache_copies_cycled": st.copies},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None},
        "path_roofline_frac": round(roof_ms / ms, 4),
        "per_call": per_call,
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = st.cpu_baseline(args.cpu_queries)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
