"""The V4-Flash attention shapes ("DeepSeek V4-Pro" card, Family: 64 query
heads, CSA top-k 512) against the oracle.  With at most 64 heads the
attention kernel splits each head block's channels over two waves (the
channel-split geometry), so these tests cover its partial-logit exchange,
both epilogues (one split per query, and split partials merged by the
combine kernel), head counts that leave a head block partly or wholly empty,
the exact-max second pass and the learned-scale parameters.  Bars as for the
other attention tests: max-abs <= 2e-2 and rel-RMS <= 5e-3 with the oracle's
indices; fp8 indexer recall >= 99.5 % with misses within 1e-3 relative."""
import math
import sys

import numpy as np
import pytest
import torch

import compressed_attention_kv_amd as cakv
import oracle
from compressed_attention_kv_amd.gen import make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _d(t):
    return t.to(DEV) if isinstance(t, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(t)).to(DEV)


def _check(out, ref, what):
    out = out.astype(np.float64)
    err = np.abs(out - ref)
    rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    say(f"  {what}: max-abs {err.max():.3e} rel-RMS {rel:.3e}")
    assert np.all(np.isfinite(out)) and err.max() <= 2e-2 and rel <= 5e-3


def _prep(kv, m, r, **kw):
    return cakv.kv_prepare(_d(kv).clone(), m=m, rope_dims=r, **kw)


def _prep_raw(raw, raw0, r, **kw):
    return cakv.kv_prepare_raw(_d(raw).clone(), np.asarray(raw0).tolist(), rope_dims=r, **kw)


def test_flash_csa_decode_128k():
    """32 queries at 128K context, 64 heads, the fp8 indexer keeping 512."""
    say("V4-Flash CSA decode 128K: indexer k=512 and sparse attention, 64 heads")
    inp = make_inputs("flash_csa_decode_128k")
    w = inp["workload"]
    codes, scale = oracle.q8_quantize(inp["k_idx"].numpy())
    scores, nvis = oracle.indexer_scores(inp["q_idx"], inp["w"], inp["q_pos"], w.m, k_code=codes, k_scale=scale)
    ref_idx = oracle.topk(scores, nvis, w.k)
    got = cakv.indexer_topk(_d(inp["q_idx"]), _d(inp["w"]), _d(codes), _d(scale), _d(inp["q_pos"]), w.m, w.k)
    got = got.cpu().numpy().reshape(ref_idx.shape)
    recalls = []
    for r in range(ref_idx.shape[0]):
        gs, rs = set(got[r].tolist()), set(ref_idx[r].tolist())
        recalls.append(len(gs & rs) / len(rs))
        kth = np.sort(scores[r].astype(np.float64))[::-1][w.k - 1]
        for j in gs ^ rs:
            assert abs(scores[r, j] - kth) <= 1e-3 * abs(kth)
    say(f"  recall {np.mean(recalls):.5f}")
    assert np.mean(recalls) >= 0.995
    idx = ref_idx.reshape(w.B, w.Q, w.k)
    kw = dict(m=w.m, n_win=w.n_win, rope_dims=w.rope_dims, rope_base=w.rope_base)
    ref, lse_ref = oracle.attention(inp["q"], inp["kv"], inp["kv_raw"], inp["raw_pos0"], inp["q_pos"], inp["sinks"],
                                    idx=idx, **kw)
    out, lse = cakv.sparse_mqa_fwd(_d(inp["q"]), _prep(inp["kv"], w.m, w.rope_dims), _d(idx),
                                   _prep_raw(inp["kv_raw"], inp["raw_pos0"], w.rope_dims), _d(inp["raw_pos0"]),
                                   _d(inp["q_pos"]), _d(inp["sinks"]), **kw)
    _check(out.float().cpu().numpy().reshape(ref.shape), ref, "sparse out bf16")
    assert np.abs(lse.cpu().numpy().reshape(lse_ref.shape) - lse_ref).max() < 1e-2


def test_flash_hca_decode_1m():
    say("V4-Flash HCA decode 1M: dense attention over 8,192 entries, 64 heads")
    inp = make_inputs("flash_hca_decode_1m")
    w = inp["workload"]
    kw = dict(m=w.m, n_win=w.n_win, rope_dims=w.rope_dims, rope_base=w.rope_base)
    ref, lse_ref = oracle.attention(inp["q"], inp["kv"], inp["kv_raw"], inp["raw_pos0"], inp["q_pos"], inp["sinks"],
                                    **kw)
    out, lse = cakv.dense_compressed_mqa_fwd(_d(inp["q"]), _prep(inp["kv"], w.m, w.rope_dims),
                                             _prep_raw(inp["kv_raw"], inp["raw_pos0"], w.rope_dims),
                                             _d(inp["raw_pos0"]), _d(inp["q_pos"]), _d(inp["sinks"]), **kw)
    _check(out.float().cpu().numpy().reshape(ref.shape), ref, "dense out bf16")
    assert np.abs(lse.cpu().numpy().reshape(lse_ref.shape) - lse_ref).max() < 1e-2


@pytest.mark.parametrize("H,BQ,odt", [(64, 256, torch.bfloat16), (64, 3, torch.float32), (40, 256, torch.float32),
                                      (40, 2, torch.bfloat16), (20, 256, torch.bfloat16), (20, 3, torch.float32),
                                      (33, 5, torch.bfloat16)])
def test_flash_head_counts_and_epilogues(H, BQ, odt):
    """Head counts up to 64 (a partly empty second head block at 40 and 33,
    an empty one at 20), one split per query (256 queries: the forward
    kernel's epilogue) or several (the partials and the combine), bf16 and
    f32 output, a -inf sink, sparse and dense calls."""
    say(f"channel split H={H} B*Q={BQ} out={odt}")
    g = torch.Generator().manual_seed(H * 1000 + BQ)
    B, Q = (2, BQ // 2) if BQ % 2 == 0 else (BQ, 1)
    D, N, R, K, m = 512, 900, 64, 128, 4
    q = torch.randn(B, Q, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    raw = torch.randn(B, R, D, generator=g).to(torch.bfloat16)
    sinks = torch.randn(H, generator=g)
    sinks[H // 3] = -math.inf
    qpos = torch.randint(4 * N - 100, 4 * N + 30, (B, Q), generator=g, dtype=torch.int32)
    qpos[0, 0] = 3  # window and sink only
    raw0 = (qpos.max(dim=1).values - R + 1).clamp(min=0).to(torch.int32)
    idx = torch.stack([torch.stack([torch.randperm(N, generator=g)[:K] for _ in range(Q)]) for _ in range(B)])
    idx = idx.sort(dim=-1).values.to(torch.int32)
    idx[:, :, ::5] = -1
    kw = dict(m=m, n_win=32, rope_dims=64)
    kvp, rawp = _prep(kv, m, 64), _prep_raw(raw, raw0, 64)
    ref, lse_ref = oracle.attention(q, kv, raw, raw0, qpos, sinks, idx=idx.numpy(), **kw)
    out, lse = cakv.sparse_mqa_fwd(_d(q), kvp, _d(idx), rawp, _d(raw0), _d(qpos), _d(sinks), out_dtype=odt, **kw)
    _check(out.float().cpu().numpy().reshape(ref.shape), ref, "sparse")
    _lse_check(lse, lse_ref)
    ref2, lse2_ref = oracle.attention(q, kv, raw, raw0, qpos, sinks, **kw)
    out2, lse2 = cakv.dense_compressed_mqa_fwd(_d(q), kvp, rawp, _d(raw0), _d(qpos), _d(sinks), out_dtype=odt, **kw)
    _check(out2.float().cpu().numpy().reshape(ref2.shape), ref2, "dense")
    _lse_check(lse2, lse2_ref)


def _lse_check(lse, lse_ref):
    """lse within 1e-2 (bf16 logits) where finite; -inf exactly where the
    oracle's is (a query with no keys and a -inf sink)."""
    lg = lse.cpu().numpy().reshape(lse_ref.shape)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lg), fin) and np.all(np.isneginf(lg[~fin]))
    assert np.abs(lg[fin] - lse_ref[fin]).max() < 1e-2


def test_flash_needle_forces_exact_max_pass():
    """A key equal to one head's query late in the sequence: that head block's
    two waves flag together and redo the key loop with the exact max."""
    say("channel split needle (second pass)")
    g = torch.Generator().manual_seed(71)
    B, Q, H, D, N = 2, 1, 64, 512, 2048
    q = torch.randn(B, Q, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    kv[0, 1900] = q[0, 0, 5]
    kv[1, 1500] = q[1, 0, 50]
    raw = torch.randn(B, 128, D, generator=g).to(torch.bfloat16)
    t = 4 * N
    qpos = torch.full((B, Q), t, dtype=torch.int32)
    raw0 = torch.full((B,), t - 127, dtype=torch.int32)
    sinks = torch.randn(H, generator=g)
    kw = dict(m=4, n_win=128, rope_dims=0)
    ref, _ = oracle.attention(q, kv, raw, raw0, qpos, sinks, **kw)
    out, _ = cakv.dense_compressed_mqa_fwd(_d(q), _prep(kv, 4, 0), _prep_raw(raw, raw0, 0), _d(raw0), _d(qpos),
                                           _d(sinks), out_dtype=torch.float32, **kw)
    _check(out.cpu().numpy().reshape(ref.shape), ref, "needle")
    assert np.abs(ref[0, 5]).max() > 0.5 and np.abs(ref[1, 50]).max() > 0.5


@pytest.mark.parametrize("BQ", [256, 4])
def test_flash_learned_scales(BQ):
    """gamma_q (the query's channel halves meet in the norm), gamma_kv,
    softmax_scale 0.05, rms_eps 1e-5 and an entry offset at 64 heads."""
    say(f"channel split with learned scales, B*Q={BQ}")
    g = torch.Generator().manual_seed(BQ + 5)
    B, Q = (2, BQ // 2)
    H, D, N, R, K, m = 64, 512, 1200, 64, 256, 4
    q = torch.randn(B, Q, H, D, generator=g).to(torch.bfloat16)
    kv = (torch.randn(B, N, D, generator=g) * 2).to(torch.bfloat16)
    raw = torch.randn(B, R, D, generator=g).to(torch.bfloat16)
    sinks = torch.randn(H, generator=g)
    gq, gk = torch.rand(D, generator=g) + 0.5, torch.rand(D, generator=g) + 0.5
    qpos = torch.randint(4 * N - 60, 4 * N + 20, (B, Q), generator=g, dtype=torch.int32)
    raw0 = (qpos.max(dim=1).values - R + 1).to(torch.int32)
    idx = torch.stack([torch.stack([torch.randperm(N, generator=g)[:K] for _ in range(Q)]) for _ in range(B)])
    idx = idx.sort(dim=-1).values.to(torch.int32)
    kw = dict(m=m, n_win=32, rope_dims=64, rope_base=10000.0, softmax_scale=0.05, rms_eps=1e-5)
    kvp = cakv.kv_prepare(_d(kv).clone(), m=m, rope_dims=64, entry_pos_offset=3, rms_eps=1e-5, gamma_kv=_d(gk))
    rawp = cakv.kv_prepare_raw(_d(raw).clone(), raw0.tolist(), rope_dims=64, rms_eps=1e-5, gamma_kv=_d(gk))
    ref, _ = oracle.attention(q, kv, raw, raw0, qpos, sinks, idx=idx.numpy(), entry_pos_offset=3, gamma_q=gq,
                              gamma_kv=gk, **kw)
    out, _ = cakv.sparse_mqa_fwd(_d(q), kvp, _d(idx), rawp, _d(raw0), _d(qpos), _d(sinks), gamma_q=_d(gq),
                                 out_dtype=torch.float32, **kw)
    _check(out.cpu().numpy().reshape(ref.shape), ref, "sparse learned scales")
