"""Pins of the CPU oracle against facts that do not come from the oracle itself:
closed forms, library routines (torch SDPA, torch's fp8 cast, numpy sorting),
the counts the pages print (tests/golden/page_counts.txt), hand-derived
values (tests/golden/indexer_canonical_order.txt), invariants and fp64
brute force on tiny inputs.  Each test names the mistake it would catch.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_counts():
    vals = {}
    with open(os.path.join(GOLDEN, "page_counts.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, value = line.split()[:2]
                vals[name] = int(value)
    return vals


# --------------------------------------------------------------------------
# O1 compression
# --------------------------------------------------------------------------

def test_compress_counts_match_pages():
    """1M tokens compress to ~262,000 CSA entries and 8,192 HCA entries."""
    g = _golden_counts()
    T = g["context_tokens"]
    x = torch.zeros(1, T, 1)
    gate = torch.zeros(1, T)
    assert oracle.kv_compress(x, gate, g["csa_ratio"]).shape[1] == g["csa_entries_at_1m"]
    assert oracle.kv_compress(x, gate, g["hca_ratio"]).shape[1] == g["hca_entries_at_1m"]
    # a partial trailing block produces no entry
    assert oracle.kv_compress(torch.zeros(1, 131, 1), torch.zeros(1, 131), 4).shape[1] == 32


def test_compress_equal_logits_is_block_mean():
    """Equal gate logits give uniform weights: the block mean (catches a dropped normaliser)."""
    rng = np.random.default_rng(1)
    x = rng.standard_normal((2, 64, 16)).astype(np.float32)
    gate = np.full((2, 64), 0.37, np.float32)
    for m in (1, 4, 16, 64):
        got = oracle.kv_compress(x, gate, m)
        want = x.astype(np.float64).reshape(2, 64 // m, m, 16).mean(axis=2)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-14)


def test_compress_known_weights():
    """Gates [0, ln 3] give weights 1/4 and 3/4 (hand-derived; catches sign of the exponent)."""
    x = np.array([[[4.0], [8.0]]], np.float32)
    gate = np.array([[0.0, math.log(3.0)]], np.float32)
    got = oracle.kv_compress(x, gate, 2)[0, 0, 0]
    w1 = 3.0 / (1.0 + 3.0)  # exp(ln 3) with ln 3 rounded to fp32 is 3 within 1e-7
    assert abs(got - (4.0 * (1 - w1) + 8.0 * w1)) < 1e-6


def test_compress_dominant_token_and_identity():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 32, 8)).astype(np.float32)
    gate = np.full((1, 32), -30.0, np.float32)
    gate[0, 2::4] = 30.0  # third token of each block dominates by e^60
    got = oracle.kv_compress(x, gate, 4)
    np.testing.assert_allclose(got[0], x[0, 2::4], rtol=1e-20, atol=1e-20)
    # m = 1 is the identity whatever the gates
    np.testing.assert_array_equal(oracle.kv_compress(x, rng.standard_normal((1, 32)).astype(np.float32), 1),
                                  x.astype(np.float64))


def test_compress_linear_and_gate_shift_invariant():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((1, 48, 8)).astype(np.float32)
    y = rng.standard_normal((1, 48, 8)).astype(np.float32)
    gate = rng.standard_normal((1, 48)).astype(np.float32)
    cx, cy = oracle.kv_compress(x, gate, 4), oracle.kv_compress(y, gate, 4)
    np.testing.assert_allclose(oracle.kv_compress(x + y, gate, 4), cx + cy, atol=1e-6)
    # constant sequence stays constant
    c = oracle.kv_compress(np.full((1, 48, 8), 2.5, np.float32), gate, 4)
    np.testing.assert_allclose(c, 2.5, rtol=1e-14)
    # adding a constant to the gate logits does not change softmax weights
    np.testing.assert_allclose(oracle.kv_compress(x, gate + 5.0, 4), cx, atol=1e-6)


def test_compress_bf16_input_exact_values():
    x = torch.randn(1, 16, 8).to(torch.bfloat16)
    gate = torch.randn(1, 16)
    a = oracle.kv_compress(x, gate, 4)
    b = oracle.kv_compress(x.float(), gate, 4)
    np.testing.assert_array_equal(a, b)


# --------------------------------------------------------------------------
# fp8 E4M3 and the per-entry quantiser
# --------------------------------------------------------------------------

def test_e4m3_decode_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = np.array([oracle.e4m3_decode(c) for c in range(256)])
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(nan, np.isnan(got))
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.nanmax(got) == 448.0


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.standard_normal(20000) * 50, rng.standard_normal(5000) * 1e-2,
                        rng.uniform(-448, 448, 5000)])
    # exact midpoints between neighbouring codes exercise ties-to-even
    mags = np.array([oracle.e4m3_decode(c) for c in range(0x7F)])
    mids = (mags[1:] + mags[:-1]) / 2
    v = np.concatenate([v, mids, -mids]).astype(np.float32)
    got = np.array([oracle.e4m3_encode(float(x)) for x in v], dtype=np.uint8)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, ref)


def test_e4m3_saturates():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(470.0) == 0x7E
    assert oracle.e4m3_encode(-1e30) == 0xFE


def test_q8_scale_rule_and_exact_dequant():
    c = np.array([[448.0, -1.0], [448.0001, 3.0], [224.0, 0.0], [0.0, 0.0], [-1e-30, 2e-31]], np.float64)
    codes, scale = oracle.q8_quantize(c)
    assert list(scale[:4]) == [1.0, 2.0, 0.5, 1.0]
    assert codes[3].tolist() == [0, 0]
    assert scale[4] == 2.0 ** -108  # 448 * 2^-109 < 1e-30 <= 448 * 2^-108
    rng = np.random.default_rng(5)
    x = rng.standard_normal((300, 128)) * rng.uniform(1e-3, 1e3, (300, 1))
    codes, scale = oracle.q8_quantize(x)
    deq = oracle.q8_dequantize(codes, scale).astype(np.float64)
    # every row uses the top of the range and stays within half a code step of the input
    assert np.all(np.abs(x).max(1) <= 448.0 * scale) and np.all(np.abs(x).max(1) > 224.0 * scale)
    step = np.maximum(2.0 ** (np.floor(np.log2(np.maximum(np.abs(x) / scale[:, None], 2.0 ** -6))) - 3),
                      2.0 ** -9) * scale[:, None]
    assert np.all(np.abs(deq - x) <= step / 2 + 1e-300)
    # dequantisation is exact in fp32: code value times a power of two
    table = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(deq, table[codes] * scale[:, None].astype(np.float64))


# --------------------------------------------------------------------------
# O2 indexer score and O3 top-k
# --------------------------------------------------------------------------

def test_indexer_canonical_fma_order_golden():
    with open(os.path.join(GOLDEN, "indexer_canonical_order.txt")) as f:
        want = [float.fromhex(ln.split()[1]) for ln in f if ln.startswith("score_hex")][0]
    q = np.array([[[[-1.0, 1.0 + 2.0 ** -12]]]], np.float32)
    k = np.array([[[1.0, 1.0 + 2.0 ** -12]]], np.float32)
    s, nv = oracle.indexer_scores(q, np.ones((1, 1, 1), np.float32), np.array([[4]], np.int32), 4, k_f32=k)
    assert nv[0] == 1 and s[0, 0] == np.float32(want)


def test_indexer_single_head_is_relu_dot_and_visibility():
    """H_I = 1, w = 1: score = ReLU(q . k); ranking equals numpy's argsort on fp64 dots."""
    rng = np.random.default_rng(6)
    N, dI, m = 500, 16, 4
    q = rng.standard_normal((1, 3, 1, dI)).astype(np.float32)
    k = rng.standard_normal((1, N, dI)).astype(np.float32)
    qpos = np.array([[4 * 400, 4 * 400 + 3, 5]], np.int32)
    s, nv = oracle.indexer_scores(q, np.ones((1, 3, 1), np.float32), qpos, m, k_f32=k)
    assert nv.tolist() == [400, 400, 1]
    assert np.all(np.isnan(s[0, 400:])) and np.all(np.isnan(s[2, 1:]))
    dots = np.maximum(k[0].astype(np.float64) @ q[0, 0, 0].astype(np.float64), 0.0)
    np.testing.assert_allclose(s[0, :400], dots[:400], rtol=1e-5, atol=1e-5)
    pos = dots[:400] > 0
    order = np.argsort(-dots[:400][pos], kind="stable")
    idx = oracle.topk(s, nv, 50)
    want = np.sort(np.flatnonzero(pos)[order[:50]])
    np.testing.assert_array_equal(idx[0], want)


def test_indexer_fp64_brute_force_and_permutation():
    rng = np.random.default_rng(7)
    B, Q, N, HI, dI, m = 2, 2, 64, 4, 8, 1
    q = rng.standard_normal((B, Q, HI, dI)).astype(np.float32)
    w = rng.standard_normal((B, Q, HI)).astype(np.float32)
    k = rng.standard_normal((B, N, dI)).astype(np.float32)
    qpos = np.full((B, Q), N, np.int32)
    s, _ = oracle.indexer_scores(q, w, qpos, m, k_f32=k)
    for b in range(B):
        for t in range(Q):
            dots = np.einsum("hd,nd->hn", q[b, t].astype(np.float64), k[b].astype(np.float64))
            ref = (w[b, t].astype(np.float64)[:, None] * np.maximum(dots, 0)).sum(0)
            scale = (np.abs(w[b, t])[:, None] * np.abs(dots)).sum(0) + 1e-30
            assert np.all(np.abs(s[b * Q + t] - ref) <= 1e-6 * scale)
    perm = rng.permutation(N)
    s2, _ = oracle.indexer_scores(q, w, qpos, m, k_f32=k[:, perm])
    np.testing.assert_array_equal(s2, s[:, perm])


def test_indexer_fp8_keys_use_exact_dequant():
    rng = np.random.default_rng(8)
    kraw = rng.standard_normal((1, 40, 16)).astype(np.float32)
    codes, scale = oracle.q8_quantize(kraw)
    deq = oracle.q8_dequantize(codes, scale)
    q = torch.randn(1, 1, 2, 16).to(torch.bfloat16)
    w = rng.standard_normal((1, 1, 2)).astype(np.float32)
    qpos = np.array([[160]], np.int32)
    a, _ = oracle.indexer_scores(q, w, qpos, 4, k_code=codes, k_scale=scale)
    b, _ = oracle.indexer_scores(q.float(), w, qpos, 4, k_f32=deq)
    np.testing.assert_array_equal(a, b)


def test_topk_matches_lexsort_with_ties():
    rng = np.random.default_rng(9)
    n, N, k = 6, 3000, 100
    s = rng.integers(-40, 40, size=(n, N)).astype(np.float32)  # many exact ties
    s[0] = 1.0  # all equal: lowest indices win
    s[1, ::2] = -0.0
    s[1, 1::2] = 0.0  # -0 and +0 compare equal
    nv = np.array([N, N, N, 57, 100, 0], np.int32)
    idx = oracle.topk(s, nv, k)
    for r in range(n):
        v = nv[r]
        order = np.lexsort((np.arange(v), -s[r, :v].astype(np.float64)))
        want = np.sort(order[:min(k, v)])
        assert np.array_equal(idx[r, :len(want)], want)
        assert np.all(idx[r, len(want):] == -1)
    assert idx[0].tolist() == list(range(k))
    assert idx[1].tolist() == list(range(k))
    assert idx[3].tolist() == list(range(57)) + [-1] * (k - 57)


def test_topk_is_associative_over_chunks():
    """Top-k of the union of per-chunk top-ks equals the global top-k."""
    rng = np.random.default_rng(10)
    N, k = 4096, 64
    s = (rng.standard_normal(N) * 3).round(1).astype(np.float32)
    full = oracle.topk(s[None], np.array([N], np.int32), k)[0]
    cand = []
    for c in range(0, N, 512):
        loc = oracle.topk(s[None, c:c + 512], np.array([512], np.int32), k)[0] + c
        cand.extend(loc.tolist())
    cand = np.array(cand)
    sub = s[cand]
    order = np.lexsort((cand, -sub.astype(np.float64)))
    np.testing.assert_array_equal(np.sort(cand[order[:k]]), full)


# --------------------------------------------------------------------------
# O4 attention
# --------------------------------------------------------------------------

def _pm1(rng, shape):
    """Entries +-1: every row already has mean square 1, so RMSNorm with eps 0 is the identity."""
    return (rng.integers(0, 2, size=shape) * 2 - 1).astype(np.float32)


def _sdpa(q, k, v, scale, causal=False):
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), is_causal=causal, scale=scale).numpy()


def test_attention_no_sink_is_textbook_softmax_attention():
    """Sink -inf, no rotation, pre-normalised rows: equals torch SDPA on K = V (fp64)."""
    rng = np.random.default_rng(11)
    H, D, N, m, win = 4, 16, 10, 4, 3
    t = 4 * N + 2
    q = _pm1(rng, (1, 1, H, D))
    kv = _pm1(rng, (1, N, D))
    raw = _pm1(rng, (1, win, D))
    sinks = np.full(H, -np.inf, np.float32)
    out, lse = oracle.attention(q, kv, raw, np.array([t - win + 1], np.int32), np.array([[t]], np.int32),
                                sinks, m=m, n_win=win, rope_dims=0, rms_eps=0.0)
    K = np.concatenate([kv[0], raw[0]]).astype(np.float64)
    ref = _sdpa(q[0, 0].astype(np.float64)[None], K[None], K[None], 1 / math.sqrt(D))[0]
    np.testing.assert_allclose(out[0], ref, atol=1e-12)
    logits = q[0, 0].astype(np.float64) @ K.T / math.sqrt(D)
    np.testing.assert_allclose(lse[0], np.log(np.exp(logits).sum(1)), atol=1e-12)


def test_attention_sink_closed_form():
    rng = np.random.default_rng(12)
    H, D, N = 6, 32, 20
    t = 4 * N
    q = rng.standard_normal((1, 1, H, D)).astype(np.float32)
    kv = rng.standard_normal((1, N, D)).astype(np.float32)
    raw = rng.standard_normal((1, 8, D)).astype(np.float32)
    common = dict(m=4, n_win=8, rope_dims=8)
    args = (q, kv, raw, np.array([t - 7], np.int32), np.array([[t]], np.int32))
    o0, l0 = oracle.attention(*args, np.full(H, -np.inf, np.float32), **common)
    z = rng.standard_normal(H).astype(np.float32) * 2
    oz, lz = oracle.attention(*args, z, **common)
    frac = 1.0 / (1.0 + np.exp(z.astype(np.float64) - l0[0]))  # 1 - sigmoid(z - lse)
    np.testing.assert_allclose(oz[0], o0[0] * frac[:, None], atol=1e-12)
    np.testing.assert_allclose(lz[0], np.logaddexp(l0[0], z.astype(np.float64)), atol=1e-12)


def test_attention_csa_with_all_entries_equals_dense():
    rng = np.random.default_rng(13)
    H, D, N, m = 4, 64, 33, 4
    t = 4 * 30 + 1  # 30 visible entries; entries 30..32 must stay invisible
    q = torch.randn(1, 1, H, D).to(torch.bfloat16)
    kv = torch.randn(1, N, D).to(torch.bfloat16)
    raw = torch.randn(1, 16, D).to(torch.bfloat16)
    sinks = rng.standard_normal(H).astype(np.float32)
    args = (q, kv, raw, np.array([t - 15], np.int32), np.array([[t]], np.int32), sinks)
    kw = dict(m=m, n_win=16, rope_dims=16)
    dense, ld = oracle.attention(*args, **kw)
    idx = np.array([[[-1] * 5 + list(range(N)) + [-1] * 4]], np.int32)  # includes invisible 30..32
    sparse, ls = oracle.attention(*args, idx=idx, **kw)
    np.testing.assert_allclose(sparse, dense, atol=1e-13)
    np.testing.assert_allclose(ls, ld, atol=1e-13)


def test_attention_m1_is_causal_mqa():
    """m = 1, window of one token, every earlier token selected, no sink, no rotation:
    standard causal multi-query attention (torch SDPA, is_causal=True)."""
    rng = np.random.default_rng(14)
    H, D, T = 3, 16, 12
    x = _pm1(rng, (1, T, D))
    q = _pm1(rng, (1, T, H, D))
    qpos = np.arange(T, dtype=np.int32)[None]
    idx = np.tile(np.arange(T, dtype=np.int32), (1, T, 1))  # entries >= t are invisible at m=1
    out, _ = oracle.attention(q, x, x, np.array([0], np.int32), qpos, np.full(H, -np.inf, np.float32),
                              idx=idx, m=1, n_win=1, rope_dims=0, rms_eps=0.0)
    K = x[0].astype(np.float64)
    ref = _sdpa(q[0].transpose(1, 0, 2).astype(np.float64), np.broadcast_to(K, (H, T, D)).copy(),
                np.broadcast_to(K, (H, T, D)).copy(), 1 / math.sqrt(D), causal=True)
    np.testing.assert_allclose(out.transpose(1, 0, 2), ref, atol=1e-12)


def test_attention_rotation_closed_forms():
    """One rotated pair (D = r = 2): the logit depends on cos((t - pi) theta_0) only, and a
    single key's output is the normalised key rotated by (pi - t)."""
    D = 2
    q = np.array([[[[1.0, 0.0]]]], np.float32)
    kv = np.array([[[0.0, 0.0]] * 3 + [[3.0, 4.0]]], np.float32)  # entry 3 at position 3*m
    raw = np.zeros((1, 1, D), np.float32)
    m, t = 5, 27
    idx = np.array([[[3]]], np.int32)
    out, lse = oracle.attention(q, kv, raw, np.array([0], np.int32), np.array([[t]], np.int32),
                                np.array([-np.inf], np.float32), idx=idx, m=m, n_win=0, rope_dims=2,
                                rms_eps=0.0)
    kn = np.array([3.0, 4.0]) / math.sqrt((9 + 16) / 2)
    ang = (3 * m - t) * 1.0  # theta_0 = base^0 = 1
    rot = np.array([kn[0] * math.cos(ang) - kn[1] * math.sin(ang), kn[0] * math.sin(ang) + kn[1] * math.cos(ang)])
    np.testing.assert_allclose(out[0, 0], rot, atol=1e-12)
    qn = np.array([math.sqrt(2), 0.0])
    np.testing.assert_allclose(lse[0, 0], (qn @ rot) / math.sqrt(2), atol=1e-12)


def test_attention_own_token_key_returns_normalised_key():
    """A single window key at the query's own position: the output is RMSNorm(v) * gamma,
    whatever the rotation (catches a wrong sign of the output rotation)."""
    rng = np.random.default_rng(15)
    D, t = 64, 1000
    v = rng.standard_normal((1, 1, D)).astype(np.float32)
    q = rng.standard_normal((1, 1, 2, D)).astype(np.float32)
    g = rng.uniform(0.5, 2, D).astype(np.float32)
    out, _ = oracle.attention(q, np.zeros((1, 1, D), np.float32), v, np.array([t], np.int32),
                              np.array([[t]], np.int32), np.full(2, -np.inf, np.float32), m=4096, n_win=1,
                              rope_dims=32, gamma_kv=g)
    vv = v[0, 0].astype(np.float64)
    want = vv / math.sqrt((vv ** 2).mean() + 1e-6) * g
    np.testing.assert_allclose(out[0, 0], want, atol=1e-12)
    np.testing.assert_allclose(out[0, 1], want, atol=1e-12)


def test_attention_relative_position_invariance():
    rng = np.random.default_rng(16)
    H, D, N, m, win = 4, 64, 40, 4, 8
    t = 4 * N + 3
    q = rng.standard_normal((1, 1, H, D)).astype(np.float32)
    kv = rng.standard_normal((1, N, D)).astype(np.float32)
    raw = rng.standard_normal((1, win, D)).astype(np.float32)
    sinks = rng.standard_normal(H).astype(np.float32)
    kw = dict(m=m, n_win=win, rope_dims=32, rope_base=50.0)
    a, la = oracle.attention(q, kv, raw, np.array([t - win + 1], np.int32), np.array([[t]], np.int32), sinks, **kw)
    for delta in (12, 1001):
        b, lb = oracle.attention(q, kv, raw, np.array([t - win + 1 + delta], np.int32),
                                 np.array([[t + delta]], np.int32), sinks, entry_pos_offset=delta, **kw)
        assert min((t + delta) // m, N) == min(t // m, N)  # the same entries stay visible
        np.testing.assert_allclose(b, a, atol=1e-9)
        np.testing.assert_allclose(lb, la, atol=1e-9)


def test_attention_no_rotation_is_position_free_and_early_rows():
    rng = np.random.default_rng(17)
    H, D, N, m, win = 2, 32, 8, 4, 4
    q = rng.standard_normal((1, 1, H, D)).astype(np.float32)
    kv = rng.standard_normal((1, N, D)).astype(np.float32)
    raw = rng.standard_normal((1, win, D)).astype(np.float32)
    sinks = rng.standard_normal(H).astype(np.float32)
    # r = 0: moving the window and the query together changes nothing
    t = 3
    a, _ = oracle.attention(q, kv, raw, np.array([0], np.int32), np.array([[t]], np.int32), sinks,
                            m=m, n_win=win, rope_dims=0)
    # t < m: no compressed entry is visible, so the cache contents do not matter
    b, _ = oracle.attention(q, kv * 100, raw, np.array([0], np.int32), np.array([[t]], np.int32), sinks,
                            m=m, n_win=win, rope_dims=0)
    np.testing.assert_array_equal(a, b)
    # with N = 0 entries the result is the window-only attention
    c, _ = oracle.attention(q, kv[:, :0], raw, np.array([0], np.int32), np.array([[t]], np.int32), sinks,
                            m=m, n_win=win, rope_dims=0)
    np.testing.assert_array_equal(a, c)
    # r = 0: moving the query and its window together changes nothing
    d, _ = oracle.attention(q, kv[:, :0], raw, np.array([5000], np.int32), np.array([[5000 + t]], np.int32),
                            sinks, m=m, n_win=win, rope_dims=0)
    np.testing.assert_allclose(d, a, atol=1e-14)


def test_attention_empty_key_set():
    D = 8
    out, lse = oracle.attention(np.ones((1, 1, 2, D), np.float32), np.zeros((1, 0, D), np.float32),
                                np.zeros((1, 1, D), np.float32), np.array([100], np.int32),
                                np.array([[5]], np.int32), np.array([-np.inf, 0.5], np.float32),
                                m=4, n_win=2, rope_dims=0)
    assert np.all(out == 0) and lse[0, 0] == -np.inf and lse[0, 1] == pytest.approx(0.5)


def test_attention_softmax_scale_and_gamma_q():
    """gamma_q = 2 everywhere doubles every logit, the same as softmax_scale = 2/sqrt(D)."""
    rng = np.random.default_rng(18)
    H, D, N = 2, 16, 12
    t = 4 * N
    args = (rng.standard_normal((1, 1, H, D)).astype(np.float32), rng.standard_normal((1, N, D)).astype(np.float32),
            rng.standard_normal((1, 4, D)).astype(np.float32), np.array([t - 3], np.int32),
            np.array([[t]], np.int32), rng.standard_normal(H).astype(np.float32))
    a, la = oracle.attention(*args, m=4, n_win=4, rope_dims=8, gamma_q=np.full(D, 2.0, np.float32))
    b, lb = oracle.attention(*args, m=4, n_win=4, rope_dims=8, softmax_scale=2.0 / math.sqrt(D))
    np.testing.assert_allclose(a, b, atol=1e-12)
    np.testing.assert_allclose(la, lb, atol=1e-12)


# --------------------------------------------------------------------------
# O5 entry preparation (the key half of the Q/K prep step)
# --------------------------------------------------------------------------

def test_kv_prepare_normalisation_closed_form():
    """No rotation: y = gamma * x / sqrt(mean(x^2) + eps) (catches a sum in place of a
    mean, a missing eps or gamma, a wrong row)."""
    rng = np.random.default_rng(30)
    B, N, D = 2, 5, 24
    x = rng.standard_normal((B, N, D)).astype(np.float32)
    g = rng.uniform(0.5, 2, D).astype(np.float32)
    y = oracle.kv_prepare(x, m=4, rope_dims=0, gamma_kv=g, rms_eps=0.25)
    xd = x.astype(np.float64)
    want = xd / np.sqrt((xd ** 2).mean(axis=-1, keepdims=True) + 0.25) * g
    np.testing.assert_allclose(y, want, rtol=1e-14, atol=1e-15)
    # a sub-range of entries is the same slice of the full result
    np.testing.assert_array_equal(oracle.kv_prepare(x, m=4, rope_dims=0, gamma_kv=g, rms_eps=0.25, j0=2, n=2),
                                  y[:, 2:4])


def test_kv_prepare_rotation_worked_example():
    """D = 6, r = 4, base 4; entry j = 3 with m = 2 and offset 1 sits at position p = 7: pair
    (2,3) turns by p * 4^0 = 7 rad, pair (4,5) by p * 4^(-1/2) = 3.5 rad, dims 0,1 stay (catches
    the wrong pairs, a wrong sign of the angle, a wrong per-pair frequency or position)."""
    x = np.array([[[0, 0, 0, 0, 0, 0]] * 3 + [[1.0, -2.0, 3.0, 4.0, -1.0, 2.0]]], np.float32)
    y = oracle.kv_prepare(x, m=2, rope_dims=4, rope_base=4.0, entry_pos_offset=1, rms_eps=0.0)[0, 3]
    s = math.sqrt((1 + 4 + 9 + 16 + 1 + 4) / 6)
    a0, a1 = 7.0, 3.5
    want = np.array([1.0, -2.0,
                     3.0 * math.cos(a0) - 4.0 * math.sin(a0), 3.0 * math.sin(a0) + 4.0 * math.cos(a0),
                     -1.0 * math.cos(a1) - 2.0 * math.sin(a1), -1.0 * math.sin(a1) + 2.0 * math.cos(a1)]) / s
    np.testing.assert_allclose(y, want, atol=1e-14)


def test_kv_prepare_pairwise_dots_depend_on_distance_only():
    """Shifting every entry's position by the same amount leaves all k_i . k_j unchanged
    while the vectors themselves change (RoPE is relative)."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((1, 9, 32)).astype(np.float32)
    kw = dict(m=4, rope_dims=16, rope_base=100.0)
    a = oracle.kv_prepare(x, **kw)[0]
    b = oracle.kv_prepare(x, entry_pos_offset=37, **kw)[0]
    assert np.abs(a - b).max() > 0.1
    np.testing.assert_allclose(a @ a.T, b @ b.T, atol=1e-11)


def test_kv_prepare_gives_the_attention_keys():
    """fp64 brute force on a tiny case: softmax attention (with the sink) over the prepared
    entries reproduces the attention oracle's log-sum-exp and its unrotated output dims.
    The query vector is prepared by the same rule at position t (m = 1, offset t)."""
    rng = np.random.default_rng(32)
    H, D, N, m, r = 3, 16, 7, 4, 8
    t = m * N + 2
    q = rng.standard_normal((1, 1, H, D)).astype(np.float32)
    kv = rng.standard_normal((1, N, D)).astype(np.float32)
    sinks = rng.standard_normal(H).astype(np.float32)
    gk = rng.uniform(0.5, 2, D).astype(np.float32)
    gq = rng.uniform(0.5, 2, D).astype(np.float32)
    kw = dict(rope_dims=r, rope_base=30.0, rms_eps=1e-6)
    out, lse = oracle.attention(q, kv, np.zeros((1, 1, D), np.float32), np.array([0], np.int32),
                                np.array([[t]], np.int32), sinks, m=m, n_win=0, entry_pos_offset=3,
                                gamma_q=gq, gamma_kv=gk, **kw)
    keys = oracle.kv_prepare(kv, m=m, entry_pos_offset=3, gamma_kv=gk, **kw)[0]
    for h in range(H):
        qh = oracle.kv_prepare(q[:, 0, h:h + 1], m=1, entry_pos_offset=t, gamma_kv=gq, **kw)[0, 0]
        lg = keys @ qh / math.sqrt(D)
        z = math.exp(sinks[h]) + np.exp(lg).sum()
        assert lse[0, h] == pytest.approx(math.log(z), abs=1e-12)
        o = (np.exp(lg)[:, None] * keys).sum(axis=0) / z
        np.testing.assert_allclose(out[0, h, :D - r], o[:D - r], atol=1e-12)


# ---------------------------------------------------------------- compression variants

def _compress_brute(x, gate, m, span):
    """numpy fp64 from the definition: entry j sums the tokens
    [max(0, (j+1)m - span), (j+1)m), each channel weighted by its own softmax
    over those tokens (a per-token gate is the same logit on every channel)."""
    import scipy.special
    x = np.asarray(x, np.float64)
    g = np.asarray(gate, np.float64)
    B, T, D = x.shape
    out = np.zeros((B, T // m, D))
    for b in range(B):
        for j in range(T // m):
            hi = (j + 1) * m
            lo = max(0, hi - span)
            gg = g[b, lo:hi] if g.ndim == 3 else np.repeat(g[b, lo:hi, None], D, axis=1)
            out[b, j] = (scipy.special.softmax(gg, axis=0) * x[b, lo:hi]).sum(axis=0)
    return out


@pytest.mark.parametrize("m", [1, 4, 128])
def test_compress_ex_plain_case_is_the_compressor(m):
    rng = np.random.default_rng(m)
    x = rng.standard_normal((2, 3 * m + 5, 16)).astype(np.float32)
    g = rng.standard_normal((2, 3 * m + 5)).astype(np.float32)
    assert np.array_equal(oracle.kv_compress_ex(x, g, m), oracle.kv_compress(x, g, m))


@pytest.mark.parametrize("m,span,per_channel", [(4, 4, True), (4, 8, False), (4, 8, True), (4, 13, True),
                                                (3, 7, False), (128, 256, True), (1, 5, True)])
def test_compress_ex_brute_force(m, span, per_channel):
    rng = np.random.default_rng(100 * m + span)
    T, D = 4 * m + 3, 12
    x = rng.standard_normal((2, T, D)).astype(np.float32)
    g = rng.standard_normal((2, T, D) if per_channel else (2, T)).astype(np.float32) * 3
    got = oracle.kv_compress_ex(x, g, m, span)
    want = _compress_brute(x, g, m, span)
    assert got.shape == (2, T // m, D)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13)


def test_compress_ex_per_channel_gate_constant_over_channels_is_per_token():
    rng = np.random.default_rng(7)
    x = torch.from_numpy(rng.standard_normal((2, 40, 8)).astype(np.float32)).to(torch.bfloat16)
    g = rng.standard_normal((2, 40)).astype(np.float32)
    g3 = np.repeat(g[:, :, None], 8, axis=2)
    for span in (4, 10):
        a = oracle.kv_compress_ex(x, g3, 4, span)
        b = oracle.kv_compress_ex(x, g, 4, span)
        assert np.array_equal(a, b)


def test_compress_ex_closed_forms():
    rng = np.random.default_rng(8)
    m, span, T, D = 4, 8, 24, 6
    x = rng.standard_normal((1, T, D)).astype(np.float32)
    # equal logits: each entry is the mean of its span (cut at token 0 for j = 0)
    out = oracle.kv_compress_ex(x, np.zeros((1, T, D), np.float32), m, span)
    assert np.allclose(out[0, 0], x[0, 0:4].astype(np.float64).mean(0), rtol=1e-14, atol=1e-15)
    for j in range(1, T // m):
        assert np.allclose(out[0, j], x[0, (j + 1) * m - span:(j + 1) * m].astype(np.float64).mean(0), rtol=1e-14,
                           atol=1e-15)
    # logits ramping by 60 per token dominate every span: channels with a rising
    # ramp take the span's newest token, channels with a falling ramp its
    # oldest (the other weights are below e^-60)
    ramp = 60.0 * np.arange(T, dtype=np.float32)[None, :, None]
    sign = np.where(np.arange(D) % 2 == 0, 1.0, -1.0).astype(np.float32)
    out = oracle.kv_compress_ex(x, ramp * sign, m, span)
    for j in range(T // m):
        newest, oldest = (j + 1) * m - 1, max(0, (j + 1) * m - span)
        for d in range(D):
            i = newest if d % 2 == 0 else oldest
            assert abs(out[0, j, d] - x[0, i, d]) <= 1e-15 * abs(x[0, i, d]) + 1e-24


def test_compress_ex_overlap_masked_to_the_block_is_plain():
    """With span = 2m and the earlier block's logits pushed to -1e4 (weights
    e^-1e4 = 0 in fp64), every entry equals the non-overlapping one."""
    rng = np.random.default_rng(9)
    m, T, D = 4, 40, 8
    x = rng.standard_normal((2, T, D)).astype(np.float32)
    g = rng.standard_normal((2, T)).astype(np.float32)
    plain = oracle.kv_compress(x, g, m)
    for j in range(T // m):
        gm = g.copy()
        gm[:, max(0, j * m - m):j * m] = -1e4
        assert np.array_equal(oracle.kv_compress_ex(x, gm, m, 2 * m)[:, j], plain[:, j])


def test_compress_ex_linear_and_per_channel_shift_invariant():
    rng = np.random.default_rng(10)
    # inputs on a coarse binary grid, so 0.5 x1 + 2 x2 and g + shift are exact in fp32
    x1 = np.round(rng.standard_normal((1, 30, 5)) * 64) / 64
    x2 = np.round(rng.standard_normal((1, 30, 5)) * 64) / 64
    g = (np.round(rng.standard_normal((1, 30, 5)) * 256) / 256).astype(np.float32)
    f = lambda x, gg: oracle.kv_compress_ex(x.astype(np.float32), gg, 3, 7)
    assert np.allclose(f(0.5 * x1 + 2 * x2, g), 0.5 * f(x1, g) + 2 * f(x2, g), rtol=1e-13, atol=1e-14)
    shift = rng.integers(-4, 5, size=(1, 1, 5)).astype(np.float32)  # a constant per channel
    assert np.allclose(f(x1, g + shift), f(x1, g), rtol=1e-13, atol=1e-14)


def test_compress_ex_counts_match_pages():
    """Entries per stride are unchanged by the overlap: 1,048,576 tokens at
    m = 4 give 262,144 entries with any span (the count the pages give)."""
    T = 1048576
    x = np.zeros((1, T, 4), np.float32)
    g = np.zeros((1, T), np.float32)
    assert oracle.kv_compress_ex(x, g, 4, 8).shape[1] == 262144
    assert oracle.kv_compress_ex(x, g, 128, 128).shape[1] == 8192
