"""Parity of the backward pass (training) against the oracle's fp64
gradients, each GPU call fed the same inputs as the oracle (the attention
backward gets the oracle's forward output and lse).  Bars, from the
arithmetic of each kernel (u = 2^-24, b = 2^-9 the bf16 rounding):
  * attention: the products run on bf16 MFMA operands (q_hat, do, P and dl
    rounded to bf16, key rows stored in bf16), about four independent
    roundings of at most b per term: rel-RMS <= 1e-2 (about 5 b) per
    gradient tensor and every element within 5e-2 of the tensor's largest
    magnitude;
  * indexer: the same ReLU decisions as the oracle (the canonical fp32
    score) and fp32 sums of at most n = K + HI + 8 terms: the worst-case
    bound n u sum|terms| (the oracle's absolute sums), plus for dw the
    score's own rounding, dI u sum_j |dS_j| sum_d |q_d k_d|;
  * kv_prepare and the compressor: fp32 chains of at most D (the RMSNorm
    dot) or 2 span + 8 operations: every element within (2 n) u of the
    row's largest gradient magnitude, n the chain length.
"""
import math
import sys

import numpy as np
import pytest
import torch

import compressed_attention_kv_amd as cakv
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = 2.0 ** -24


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _d(t):
    return t.to(DEV) if isinstance(t, torch.Tensor) else torch.from_numpy(np.ascontiguousarray(t)).to(DEV)


def _grad_check(got, ref, what, rel_bar=1e-2, max_frac=5e-2):
    got = got.astype(np.float64)
    err = np.abs(got - ref)
    scale = np.abs(ref).max()
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300)
    say(f"  {what}: rel-RMS {rel:.2e}, worst {err.max() / max(scale, 1e-300):.2e} of the largest magnitude")
    assert np.all(np.isfinite(got))
    assert rel <= rel_bar and err.max() <= max_frac * scale


def _attn_case(seed, B, Q, H, N, R, K, sparse, n_win=32, gamma=True, m=4):
    g = torch.Generator().manual_seed(seed)
    D = 512
    q = torch.randn(B, Q, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    raw = torch.randn(B, R, D, generator=g).to(torch.bfloat16)
    sinks = torch.randn(H, generator=g)
    sinks[H // 2] = -math.inf
    gq = torch.rand(D, generator=g) + 0.5 if gamma else None
    qpos = torch.randint(m * N - 40, m * N + 20, (B, Q), generator=g, dtype=torch.int32)
    raw0 = (qpos.max(dim=1).values - R + 1).clamp(min=0).to(torch.int32)
    idx = None
    if sparse:
        idx = torch.stack([torch.stack([torch.randperm(N, generator=g)[:K] for _ in range(Q)]) for _ in range(B)])
        idx = idx.to(torch.int32)
        idx[:, :, ::9] = -1
    dout = torch.randn(B, Q, H, D, generator=g)
    kw = dict(m=m, n_win=n_win, rope_dims=64, rope_base=10000.0, softmax_scale=0.0, rms_eps=1e-6)
    return dict(q=q, kv=kv, raw=raw, sinks=sinks, gq=gq, qpos=qpos, raw0=raw0, idx=idx, dout=dout, kw=kw)


@pytest.mark.parametrize("name,B,Q,H,N,R,K,sparse", [
    ("sparse, 4 queries (key splits)", 2, 2, 128, 600, 64, 128, True),
    ("dense, 2 queries (key splits)", 2, 1, 128, 300, 64, 0, False),
    ("sparse, 256 queries (one split)", 2, 128, 32, 200, 160, 48, True),
    ("sparse, 64 heads", 2, 2, 64, 500, 64, 256, True),
    ("dense, 40 heads (padded head block)", 1, 3, 40, 400, 48, 0, False),
    ("sparse, 2,100 selected (dq reads the indices from memory)", 1, 1, 128, 3000, 64, 2100, True),
])
def test_attention_backward(name, B, Q, H, N, R, K, sparse):
    say(f"attention backward: {name}")
    c = _attn_case(sum(map(ord, name)), B, Q, H, N, R, K, sparse)
    kw = c["kw"]
    idx_np = None if c["idx"] is None else c["idx"].numpy()
    out_ref, lse_ref = oracle.attention(c["q"], c["kv"], c["raw"], c["raw0"], c["qpos"], c["sinks"], idx=idx_np,
                                        gamma_q=c["gq"], **kw)
    ref = oracle.attention_bwd(c["q"], c["kv"], c["raw"], c["raw0"], c["qpos"], c["sinks"], c["dout"], idx=idx_np,
                               gamma_q=c["gq"], **kw)
    kvp = cakv.kv_prepare(_d(c["kv"]).clone(), m=kw["m"], rope_dims=kw["rope_dims"])
    rawp = cakv.kv_prepare_raw(_d(c["raw"]).clone(), c["raw0"].tolist(), rope_dims=kw["rope_dims"])
    out = torch.from_numpy(out_ref.astype(np.float32)).view(B, Q, H, 512)
    lse = torch.from_numpy(lse_ref.astype(np.float32)).view(B, Q, H)
    got = cakv.mqa_bwd(_d(c["q"]), kvp, None if c["idx"] is None else _d(c["idx"]), rawp, _d(c["raw0"]),
                       _d(c["qpos"]), _d(c["sinks"]), _d(out), _d(lse), _d(c["dout"]), gamma_q=_d(c["gq"]), **kw)
    _grad_check(got["dq"].cpu().numpy().reshape(ref["dq"].shape), ref["dq"], "dq")
    _grad_check(got["dkv_c"].cpu().numpy(), ref["dkhat_c"], "dkv_c (prepared cache rows)")
    _grad_check(got["dkv_raw"].cpu().numpy(), ref["dkhat_raw"], "dkv_raw (prepared window rows)")
    _grad_check(got["dsinks"].cpu().numpy(), ref["dsinks"], "dsinks")
    _grad_check(got["dgamma_q"].cpu().numpy(), ref["dgamma_q"], "dgamma_q")
    assert got["dsinks"][H // 2].item() == 0.0  # a -inf sink has no gradient


def test_attention_backward_degenerate_queries():
    """Four queries over raw rows that hold positions 0 .. 7: position 0 (no
    compressed entry yet, its own window row only), position 5 with every
    selection slot empty (window only), position 200 with an empty selection
    and a window outside the raw rows (no key at all), position 150 (selected
    entries only, some of them not yet visible); half the sinks are -inf.  The
    keyless query's gradients are exactly zero on every head (output 0, lse
    -inf on the heads with a -inf sink, the sink's own on the others), a -inf
    sink has no gradient, and the rest match the oracle."""
    say("attention backward, degenerate queries")
    g = torch.Generator().manual_seed(31)
    B, Q, H, N, R, K, D = 1, 4, 32, 40, 8, 16, 512
    q = torch.randn(B, Q, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    raw = torch.randn(B, R, D, generator=g).to(torch.bfloat16)
    sinks = torch.randn(H, generator=g)
    sinks[::2] = -math.inf
    qpos = torch.tensor([[0, 5, 200, 150]], dtype=torch.int32)
    raw0 = torch.tensor([0], dtype=torch.int32)
    idx = torch.stack([torch.randperm(N, generator=g)[:K] for _ in range(Q)]).view(B, Q, K).to(torch.int32)
    idx[0, 1:3] = -1
    dout = torch.randn(B, Q, H, D, generator=g)
    kw = dict(m=4, n_win=4, rope_dims=64, rope_base=10000.0, softmax_scale=0.0, rms_eps=1e-6)
    out_ref, lse_ref = oracle.attention(q, kv, raw, raw0, qpos, sinks, idx=idx.numpy(), **kw)
    ref = oracle.attention_bwd(q, kv, raw, raw0, qpos, sinks, dout, idx=idx.numpy(), **kw)
    assert np.all(np.isneginf(lse_ref[2, ::2])) and np.all(out_ref[2] == 0.0)
    assert np.all(ref["dq"][0, 2] == 0.0)
    kvp = cakv.kv_prepare(_d(kv).clone(), m=4, rope_dims=64)
    rawp = cakv.kv_prepare_raw(_d(raw).clone(), raw0.tolist(), rope_dims=64)
    out = torch.from_numpy(out_ref.astype(np.float32)).view(B, Q, H, D)
    lse = torch.from_numpy(lse_ref.astype(np.float32)).view(B, Q, H)
    got = cakv.mqa_bwd(_d(q), kvp, _d(idx), rawp, _d(raw0), _d(qpos), _d(sinks), _d(out), _d(lse), _d(dout), **kw)
    dq = got["dq"].cpu().numpy().reshape(ref["dq"].shape)
    assert np.all(np.isfinite(dq)) and np.all(dq[0, 2] == 0.0)
    live = [0, 1, 3]
    _grad_check(dq[0, live], ref["dq"][0, live], "dq (queries with keys)")
    _grad_check(got["dkv_c"].cpu().numpy(), ref["dkhat_c"], "dkv_c (position 150's entries)")
    _grad_check(got["dkv_raw"].cpu().numpy(), ref["dkhat_raw"], "dkv_raw (positions 0 .. 5)")
    ds = got["dsinks"].cpu().numpy()
    assert np.all(ds[::2] == 0.0)
    _grad_check(ds[1::2], ref["dsinks"][1::2], "dsinks (finite sinks)")


def test_attention_backward_ring_window():
    """The window read from a ring (row p mod R holds position p), as the
    streaming decode step keeps it: the window rows' gradient lands in the
    ring's rows."""
    say("attention backward, ring-mode window")
    B, Q, H, N, R, K = 2, 1, 128, 400, 128, 64
    c = _attn_case(77, B, Q, H, N, R, K, True, n_win=128)
    kw = c["kw"]
    # a linear window for the oracle: rows raw0 .. raw0+R-1; the ring holds
    # position p at row p mod R
    ring = torch.empty_like(c["raw"])
    for b in range(B):
        p = int(c["raw0"][b]) + torch.arange(R)
        ring[b, p % R] = c["raw"][b]
    out_ref, lse_ref = oracle.attention(c["q"], c["kv"], c["raw"], c["raw0"], c["qpos"], c["sinks"],
                                        idx=c["idx"].numpy(), gamma_q=c["gq"], **kw)
    ref = oracle.attention_bwd(c["q"], c["kv"], c["raw"], c["raw0"], c["qpos"], c["sinks"], c["dout"],
                               idx=c["idx"].numpy(), gamma_q=c["gq"], **kw)
    kvp = cakv.kv_prepare(_d(c["kv"]).clone(), m=kw["m"], rope_dims=kw["rope_dims"])
    ringp = _d(ring).clone()
    for b in range(B):  # each ring row prepared at its position
        p0 = int(c["raw0"][b])
        rows = (p0 + torch.arange(R)) % R
        prepared = cakv.kv_prepare(_d(c["raw"][b:b + 1]).clone(), m=1, rope_dims=kw["rope_dims"], entry_pos_offset=p0)
        ringp[b, rows.to(DEV)] = prepared[0]
    out = torch.from_numpy(out_ref.astype(np.float32)).view(B, Q, H, 512)
    lse = torch.from_numpy(lse_ref.astype(np.float32)).view(B, Q, H)
    got = cakv.mqa_bwd(_d(c["q"]), kvp, _d(c["idx"]), ringp, None, _d(c["qpos"]), _d(c["sinks"]), _d(out), _d(lse),
                       _d(c["dout"]), gamma_q=_d(c["gq"]), raw_ring=True, **kw)
    dring = got["dkv_raw"].cpu().numpy()
    dlin = np.stack([dring[b][(int(c["raw0"][b]) + np.arange(R)) % R] for b in range(B)])
    _grad_check(dlin, ref["dkhat_raw"], "dkv_raw through the ring")
    _grad_check(got["dq"].cpu().numpy().reshape(ref["dq"].shape), ref["dq"], "dq")


@pytest.mark.parametrize("dtype,gamma", [("bf16", True), ("f32", False)])
def test_kv_prepare_backward(dtype, gamma):
    say(f"kv_prepare backward {dtype} gamma={gamma}")
    g = torch.Generator().manual_seed(9)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, N, D, r, m, off, j0, n = 2, 300, 512, 64, 4, 3, 17, 250
    x = (torch.randn(B, N, D, generator=g) * 3).to(tdt)
    gk = torch.rand(D, generator=g) + 0.5 if gamma else None
    dy = torch.randn(B, N, D, generator=g)
    kw = dict(m=m, rope_dims=r, entry_pos_offset=off, rms_eps=1e-6, j0=j0, n=n)
    ref_dx, ref_dg = oracle.kv_prepare_bwd(x, dy[:, j0:j0 + n].numpy(), gamma_kv=gk, **kw)
    dgk = torch.zeros(D, dtype=torch.float32, device=DEV)
    dx = cakv.kv_prepare_bwd(_d(x), _d(dy), gamma_kv=None if gk is None else _d(gk), dgamma_kv=dgk, **kw)
    got = dx.cpu().numpy()
    assert np.all(got[:, :j0] == 0) and np.all(got[:, j0 + n:] == 0)  # rows outside the range untouched
    got = got[:, j0:j0 + n]
    bound = 2 * D * U * np.abs(ref_dx).max(axis=-1, keepdims=True)
    say(f"  dx worst error / bound {np.max(np.abs(got - ref_dx) / bound):.3f}")
    assert np.all(np.abs(got - ref_dx) <= bound)
    if gamma:  # sums over B*n rows of D-term products
        gd = dgk.cpu().numpy()
        assert np.all(np.abs(gd - ref_dg) <= 2 * (B * n + D) * U * np.abs(ref_dg).max())


@pytest.mark.parametrize("m,span,per_channel,dtype", [(4, 4, False, "bf16"), (4, 8, True, "bf16"),
                                                      (128, 128, False, "bf16"), (4, 12, False, "f32"),
                                                      (128, 256, True, "f32")])
def test_kv_compress_backward(m, span, per_channel, dtype):
    say(f"kv_compress backward m={m} span={span} per_channel={per_channel} {dtype}")
    g = torch.Generator().manual_seed(m + span)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    B, T, D = 2, 8 * m + 5 if m < 128 else 600, 128
    x = torch.randn(B, T, D, generator=g).to(tdt)
    gate = torch.randn((B, T, D) if per_channel else (B, T), generator=g) * 2
    dc = torch.randn(B, T // m, D, generator=g)
    ref_dx, ref_dg = oracle.kv_compress_bwd(x, gate, m, dc.numpy(), span)
    dx, dg = cakv.kv_compress_bwd(_d(x), _d(gate), m, _d(dc), span)
    n = 2 * span + 8 + (D if not per_channel else 0)  # per-token gates also sum over the channels
    for what, got, ref in (("dx", dx.cpu().numpy(), ref_dx), ("dgate", dg.cpu().numpy(), ref_dg)):
        rows = np.abs(ref).max(axis=-1, keepdims=True) if ref.ndim == 3 else np.abs(ref).max(axis=-1, keepdims=True)
        bound = 2 * n * U * rows + 1e-30
        say(f"  {what} worst error / bound {np.max(np.abs(got - ref) / bound):.3f}")
        assert np.all(np.abs(got - ref) <= bound)


# (B, Q, HI, dI, N, K): the V4 indexer shape, then ragged ones (odd head
# counts, head dims that fill part of a 32-wide tile, a partial last block of
# 128 slots, a query before the first entry)
INDEXER_BWD_SHAPES = [(2, 3, 64, 128, 3000, 512), (2, 2, 5, 24, 700, 300), (1, 3, 33, 72, 500, 130)]


@pytest.mark.parametrize("shape", INDEXER_BWD_SHAPES, ids=["v4", "ragged_small", "ragged_mid"])
@pytest.mark.parametrize("mode", ["f32", "fp8"])
def test_indexer_backward(mode, shape):
    say(f"indexer backward {mode} {shape}")
    rng = np.random.default_rng(42)
    B, Q, HI, dI, N, K = shape
    m = 4
    q = rng.standard_normal((B, Q, HI, dI)).astype(np.float32)
    w = rng.standard_normal((B, Q, HI)).astype(np.float32)
    keys = rng.standard_normal((B, N, dI)).astype(np.float32)
    qpos = np.full((B, Q), 4 * N, dtype=np.int32)
    qpos[0, 1] = 4 * (N // 3)  # fewer visible entries
    if shape != INDEXER_BWD_SHAPES[0]:
        qpos[-1, 0] = -1  # no visible entry: zero gradients
    idx = np.stack([np.stack([rng.permutation(N)[:K] for _ in range(Q)]) for _ in range(B)]).astype(np.int32)
    idx[:, :, ::11] = -1
    dS = rng.standard_normal((B, Q, K)).astype(np.float32)
    if mode == "fp8":
        qt = torch.from_numpy(q).to(torch.bfloat16)
        codes, scale = oracle.q8_quantize(keys)
        kk = dict(k_code=codes, k_scale=scale)
        kdev, sdev = _d(codes).view(torch.float8_e4m3fn), _d(scale)
        kf = oracle.q8_dequantize(codes, scale)
        qf = qt.float().numpy()
    else:
        qt = torch.from_numpy(q)
        kk = dict(k_f32=keys)
        kdev, sdev = _d(keys), None
        kf, qf = keys, q
    ref = oracle.indexer_bwd(qt, w, qpos, m, idx, dS, **kk)
    absr = oracle.indexer_bwd(qt, w, qpos, m, idx, dS, absolute=True, **kk)
    got = cakv.indexer_bwd(_d(qt), _d(w), kdev, sdev, _d(qpos), _d(idx), _d(dS), m)
    n = K + HI + Q + 8
    # dw also carries the fp32 score's rounding: dI u sum_j |dS_j| sum_d |q_d k_d|
    extra = np.zeros((B, Q, HI))
    for b in range(B):
        for i in range(Q):
            nv = min(int(qpos[b, i]) // m, N)
            sel = [(s, j) for s, j in enumerate(idx[b, i]) if 0 <= j < nv]
            js = np.array([j for _, j in sel], dtype=np.int64)
            ds = np.abs(np.array([dS[b, i, s] for s, _ in sel], dtype=np.float64))
            extra[b, i] = dI * U * (np.abs(qf[b, i]).astype(np.float64) @ np.abs(kf[b, js]).T.astype(np.float64)) @ ds
    for what, g_, r_, a_, ex in (("dq", got[0], ref[0], absr[0], 0.0), ("dw", got[1], ref[1], absr[1], extra),
                                 ("dk", got[2], ref[2], absr[2], 0.0)):
        g_ = g_.cpu().numpy().astype(np.float64)
        bound = n * U * a_ + ex + 1e-30
        say(f"  {what}: worst error / bound {np.max(np.abs(g_ - r_) / bound):.3f}")
        assert np.all(np.abs(g_ - r_) <= bound)
