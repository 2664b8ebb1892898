"""Parity of the HIP path against the CPU oracle, element by element, on the
same seeded inputs.  Bars (the method's stated tolerances):
  * kv_compress: the a-priori bound of the kernel's fp32 arithmetic,
    (2m + 10) * 2^-24 * sum_i a_i |x_i| per element (a_i the block's softmax
    weights; the oracle gives the sum exactly by compressing |x|), plus one
    bf16 ulp of the result for bf16 output; fp8 within one E4M3 step of the
    oracle's dequantised value (same scale except at an exponent boundary);
  * indexer_topk: indices bit-exact in fp32 mode; fp8 mode recall >= 99.5 %
    with every miss within 1e-3 relative of the k-th best score;
  * kv_prepare: bf16 within one bf16 ulp of the fp64 result plus 1e-6 of the
    row scale, f32 within 2e-6 relative to the row scale;
  * attention (fed the oracle's indices): max-abs <= 2e-2 and
    rel-RMS = ||o - o_ref|| / ||o_ref|| <= 5e-3.  The GPU side reads key rows
    (compressed entries and window rows) prepared by its own kv_prepare; the
    oracle attends over the raw rows.
"""
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


def _bf16_ulp(x):
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _compress_bound(x, gate, m, ref, bf16_out):
    """Error bound of kv_compress's fp32 arithmetic, derived from its steps:
    the weights e_i = exp(g_i - max) (relative error <= 2u each, u = 2^-24),
    their sum over m terms ((m - 1) u), the fma chain sum_i e_i x_i (m u of
    sum_i e_i |x_i|), then 1/z and the product (2u).  Together at most
    (2m + 10) u * sum_i a_i |x_i| per element, an absolute bound that also
    holds where the sum cancels to near zero.  bf16 output adds the rounding
    of the fp32 result: half an ulp at the result's own binade, at most one
    ulp of the exact value."""
    xa = x.abs() if isinstance(x, torch.Tensor) else np.abs(x)
    sabs = oracle.kv_compress(xa, gate, m)  # sum_i a_i |x_i|, fp64
    bound = (2 * m + 10) * 2.0 ** -24 * sabs
    return bound + _bf16_ulp(ref) if bf16_out else bound


# ------------------------------------------------------------------ kv_compress

@pytest.mark.parametrize("dtype,D,m,T", [("f32", 128, 4, 2048), ("f32", 32, 4, 2048), ("bf16", 512, 4, 8192 + 7),
                                         ("bf16", 512, 128, 8192 + 100), ("bf16", 512, 1, 64)])
def test_kv_compress(dtype, D, m, T):
    say(f"kv_compress {dtype} D={D} m={m} T={T}")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    g = torch.Generator().manual_seed(D * 7 + m)
    x = torch.randn(2, T, D, generator=g).to(tdt)
    gate = torch.randn(2, T, generator=g) * 2
    ref = oracle.kv_compress(x, gate, m)
    out = cakv.kv_compress(_d(x), _d(gate), m, tdt).float().cpu().numpy()
    assert out.shape == ref.shape
    err = np.abs(out - ref)
    bound = _compress_bound(x, gate, m, ref, dtype == "bf16")
    say(f"  worst error / bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound)


@pytest.mark.parametrize("T,m", [(8192 + 3, 4), (512, 1)])
def test_kv_compress_fp8(T, m):
    say(f"kv_compress fp8 T={T} m={m}")
    g = torch.Generator().manual_seed(11)
    x = torch.randn(2, T, 128, generator=g).to(torch.bfloat16)
    x[0, :m] *= 1e-3  # a small-magnitude entry
    x[1, 4 * m: 5 * m] = 0  # an all-zero entry
    gate = torch.randn(2, T, generator=g)
    c = oracle.kv_compress(x, gate, m)
    codes_ref, scale_ref = oracle.q8_quantize(c)
    out, scale = cakv.kv_compress(_d(x), _d(gate), m, torch.float8_e4m3fn)
    codes = out.view(torch.uint8).cpu().numpy()
    scale = scale.cpu().numpy()
    deq = oracle.q8_dequantize(codes, scale).astype(np.float64)
    deq_ref = oracle.q8_dequantize(codes_ref, scale_ref).astype(np.float64)
    same = scale == scale_ref
    assert same.mean() > 0.999  # only entries whose max sits on a power-of-two boundary may differ
    assert np.all(np.isin(scale[~same] / scale_ref[~same], [0.5, 2.0]))
    step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(deq_ref) / scale_ref[..., None], 2.0 ** -6))) - 3)
    step = np.maximum(step, 2.0 ** -9) * np.maximum(scale, scale_ref)[..., None]
    assert np.all(np.abs(deq - deq_ref) <= step * 1.0001)
    assert (codes == codes_ref).mean() > 0.999
    assert np.all(scale[1, 4] == 1.0) and np.all(codes[1, 4] == 0)


# ------------------------------------------------------------------ indexer

def _indexer_inputs(name, only=None, **over):
    inp = make_inputs(name, only=only, **over)
    w = inp["workload"]
    if w.prefill:
        keys = oracle.kv_compress(inp["k_idx"], inp["k_gate"], w.m)
    else:
        keys = inp["k_idx"].numpy()
    return inp, w, keys


def test_indexer_fp32_bit_exact_tiny_layer():
    say("indexer fp32 tiny layer (2048 queries, 512 entries, k=64)")
    inp, w, keys = _indexer_inputs("tiny_csa_f32")
    keys = keys.astype(np.float32)
    ref = oracle.indexer_topk(inp["q_idx"], inp["w"], inp["q_pos"], w.m, w.k, k_f32=keys)
    got = cakv.indexer_topk(_d(inp["q_idx"]), _d(inp["w"]), _d(keys), None, _d(inp["q_pos"]), w.m, w.k)
    got = got.cpu().numpy().reshape(ref.shape)
    assert np.array_equal(got, ref)
    assert (ref == -1).any(axis=1).sum() >= 256  # rows with fewer visible entries than k


@pytest.mark.parametrize("N,k,Q", [(3000, 64, 8), (70000, 1024, 2), (20000, 4096, 2)])  # k = 4096: the largest
def test_indexer_fp32_bit_exact_sizes(N, k, Q):
    say(f"indexer fp32 N={N} k={k}")
    rng = np.random.default_rng(N)
    B, HI, dI, m = 2, 8, 32, 4
    q = rng.standard_normal((B, Q, HI, dI)).astype(np.float32)
    wgt = rng.standard_normal((B, Q, HI)).astype(np.float32)
    keys = rng.standard_normal((B, N, dI)).astype(np.float32)
    keys[0, 100:200] = keys[0, 50]  # exact ties
    qpos = rng.integers(0, 4 * N + 50, size=(B, Q)).astype(np.int32)
    qpos[0, 0] = 4 * N
    ref = oracle.indexer_topk(q, wgt, qpos, m, k, k_f32=keys)
    got = cakv.indexer_topk(_d(q), _d(wgt), _d(keys), None, _d(qpos), m, k).cpu().numpy().reshape(ref.shape)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("tied", [3000, 5000, 10000])
def test_indexer_fp32_tied_block_at_threshold(tied):
    """A block of entries with one exact score straddles the k-th place: the
    tie at the boundary is broken by the lower index.  The tied keys share
    both histogram levels, so each size takes another select path: 3,000 are
    ranked by counting in LDS, 5,000 (more than the 4,096 ranked in LDS, fewer
    than the 8,192 listed) by the radix select over the listed entries, and
    10,000 (more than are listed) by the radix select over the whole key
    array."""
    say(f"indexer fp32 tied block {tied}")
    rng = np.random.default_rng(tied)
    B, Q, HI, dI, m, N, k = 1, 2, 8, 32, 4, 20000, 1024
    q = rng.standard_normal((B, Q, HI, dI)).astype(np.float32)
    wgt = np.abs(rng.standard_normal((B, Q, HI))).astype(np.float32)
    keys = rng.standard_normal((B, N, dI)).astype(np.float32)
    qpos = np.full((B, Q), 4 * N, dtype=np.int32)
    q[0, 1] = q[0, 0]
    wgt[0, 1] = wgt[0, 0]
    scores, _ = oracle.indexer_scores(q, wgt, qpos, m, k_f32=keys)
    j700 = int(np.argsort(-scores[0].astype(np.float64), kind="stable")[700])
    pos = rng.choice(N, size=tied, replace=False)
    keys[0, pos] = keys[0, j700]
    ref = oracle.indexer_topk(q, wgt, qpos, m, k, k_f32=keys)
    got = cakv.indexer_topk(_d(q), _d(wgt), _d(keys), None, _d(qpos), m, k).cpu().numpy().reshape(ref.shape)
    assert np.array_equal(got, ref)


def _recall_check(got, ref, scores, nvis, k):
    recalls, worst_gap = [], 0.0
    for r in range(ref.shape[0]):
        rs = set(ref[r][ref[r] >= 0].tolist())
        gs = got[r][got[r] >= 0]
        assert len(set(gs.tolist())) == len(gs) == len(rs)
        assert np.all(np.diff(gs) > 0) and np.all(gs < nvis[r])
        recalls.append(len(rs & set(gs.tolist())) / max(len(rs), 1))
        s = scores[r, :nvis[r]].astype(np.float64)
        kth = np.sort(s)[::-1][min(k, nvis[r]) - 1]
        for j in rs - set(gs.tolist()):
            gap = abs(s[j] - kth) / abs(kth)
            worst_gap = max(worst_gap, gap)
        for j in set(gs.tolist()) - rs:
            worst_gap = max(worst_gap, abs(s[j] - kth) / abs(kth))
    return float(np.mean(recalls)), worst_gap


@pytest.mark.parametrize("name,over", [("csa_decode_128k", dict(B=4)), ("csa_decode_128k", {}),
                                       ("csa_decode_1m", {})])
def test_indexer_fp8_recall(name, over):
    say(f"indexer fp8 {name} {over}")
    inp, w, keys = _indexer_inputs(name, only={"k_idx", "q_idx", "w"}, **over)
    codes, scale = oracle.q8_quantize(keys)
    scores, nvis = oracle.indexer_scores(inp["q_idx"], inp["w"], inp["q_pos"], w.m, k_code=codes, k_scale=scale)
    ref = oracle.topk(scores, nvis, w.k)
    got = cakv.indexer_topk(_d(inp["q_idx"]), _d(inp["w"]), _d(codes), _d(scale), _d(inp["q_pos"]), w.m, w.k)
    got = got.cpu().numpy().reshape(ref.shape)
    recall, gap = _recall_check(got, ref, scores, nvis, w.k)
    say(f"  recall {recall:.5f} worst relative gap of a swapped entry {gap:.2e}")
    assert recall >= 0.995 and gap <= 1e-3


@pytest.mark.parametrize("N,k,HI,dI", [(32768 + 77, 1024, 64, 128), (5000, 64, 64, 128), (9000, 512, 32, 128),
                                        (7000 + 5, 256, 64, 64), (3000, 128, 32, 64)])
def test_indexer_fp8_whole_line_loads_match(N, k, HI, dI):
    """With one query per sequence the fp8 score kernel loads whole cache
    lines and transposes them within lane quads (128-dim keys) or loads each
    lane's chunks directly (64-dim keys); with several it first packs the
    keys so that each load instruction reads 1 KiB of consecutive bytes.  The
    same bytes reach the same lanes, so identical indices: two sequences
    holding the same keys with one query each against one sequence with both
    queries (a ragged entry count, a query with fewer visible entries than
    k; 64 and 32 indexer heads, two or one head tiles per wave)."""
    say(f"indexer fp8 whole-line and packed loads, N={N} k={k} HI={HI} dI={dI}")
    rng = np.random.default_rng(N + k)
    m = 4
    keys = rng.standard_normal((1, N, dI)).astype(np.float32)
    codes, scale = oracle.q8_quantize(keys)
    q = torch.from_numpy(rng.standard_normal((1, 2, HI, dI)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.standard_normal((1, 2, HI)).astype(np.float32))
    qpos = np.array([[m * N + 3, m * (k // 2) + 1]], dtype=np.int32)
    shared = cakv.indexer_topk(_d(q), _d(w), _d(codes), _d(scale), _d(qpos), m, k).cpu().numpy().reshape(2, k)
    q1 = q.view(2, 1, HI, dI)
    sep = cakv.indexer_topk(_d(q1), _d(w.view(2, 1, HI)), _d(np.concatenate([codes, codes])),
                            _d(np.concatenate([scale, scale])), _d(qpos.reshape(2, 1)), m, k).cpu().numpy().reshape(2, k)
    assert np.array_equal(sep, shared)
    assert (shared[1] == -1).sum() == k - k // 2


@pytest.mark.parametrize("tied", [0, 3000, 5000, 10000])
def test_indexer_fp8_fused_refine_matches(tied):
    """With 512 or more queries the fp8 score grid has one workgroup per
    query, and that workgroup does the refine pass's work itself (histogram
    threshold from its own LDS, both levels written without atomics); with
    fewer queries the score, clearing and refine kernels run apart.  The
    scores are the same arithmetic, so the indices must be identical: 512
    queries alternating between two (query, position) pairs against one call
    with the two pairs.  A block of rows copied from one near the k-th place
    gives a tie at the threshold of each size that takes another select path
    (ranked by counting, radix select over the listed entries, radix select
    over the whole key array)."""
    say(f"indexer fp8 fused refine, tied block {tied}")
    rng = np.random.default_rng(77 + tied)
    HI, dI, m, N, k = 64, 128, 4, 20000 + 13, 1024
    keys = rng.standard_normal((1, N, dI)).astype(np.float32)
    codes, scale = oracle.q8_quantize(keys)
    q2 = rng.standard_normal((1, 2, HI, dI)).astype(np.float32)
    w2 = np.abs(rng.standard_normal((1, 2, HI))).astype(np.float32)
    pos2 = np.array([[m * N + 2, m * (N // 3) + 1]], dtype=np.int32)
    if tied:
        scores, _ = oracle.indexer_scores(torch.from_numpy(q2).to(torch.bfloat16).float().numpy(), w2, pos2, m,
                                          k_code=codes, k_scale=scale)
        j700 = int(np.argsort(-scores[0].astype(np.float64), kind="stable")[700])
        at = rng.choice(N, size=tied, replace=False)
        codes[0, at] = codes[0, j700]
        scale[0, at] = scale[0, j700]
    qb = torch.from_numpy(q2).to(torch.bfloat16)
    ref = cakv.indexer_topk(_d(qb), _d(w2), _d(codes), _d(scale), _d(pos2), m, k).cpu().numpy().reshape(2, k)
    sel = np.arange(512) % 2
    qm = qb[:, sel].contiguous()
    got = cakv.indexer_topk(_d(qm), _d(w2[:, sel]), _d(codes), _d(scale), _d(pos2[:, sel]), m, k)
    got = got.cpu().numpy().reshape(512, k)
    assert np.array_equal(got, ref[sel])
    assert (ref[0] >= 0).all() and (ref[1] >= 0).all()


@pytest.mark.parametrize("N,Q", [(40, 1), (100, 3), (128, 2), (129, 1), (129, 4)])
def test_indexer_fp8_small_key_arrays(N, Q):
    """Key arrays of at most a few 128-entry granules: one score workgroup per
    query (the refine work inside the score kernel, also with one query per
    sequence), and for several queries per sequence the pack pass over fewer
    than five 32-entry groups with a ragged last one.  Against the oracle on
    the same dequantised keys (recall and the gap of any swapped entry), and
    rows whose queries see fewer entries than k are the identity."""
    say(f"indexer fp8 small key arrays N={N} Q={Q}")
    rng = np.random.default_rng(1000 * N + Q)
    B, HI, dI, m, k = 2, 64, 128, 4, 16
    keys = rng.standard_normal((B, N, dI)).astype(np.float32)
    codes, scale = oracle.q8_quantize(keys)
    q = torch.from_numpy(rng.standard_normal((B, Q, HI, dI)).astype(np.float32)).to(torch.bfloat16)
    w = rng.standard_normal((B, Q, HI)).astype(np.float32)
    pos = rng.integers(m * (k + 1), m * N + 3, size=(B, Q)).astype(np.int32)
    pos[0, 0] = m * N
    pos[B - 1, Q - 1] = m * (k // 2) + 1  # fewer visible entries than k
    scores, nvis = oracle.indexer_scores(q.float().numpy(), w, pos, m, k_code=codes, k_scale=scale)
    ref = oracle.topk(scores, nvis, k)
    got = cakv.indexer_topk(_d(q), _d(w), _d(codes), _d(scale), _d(pos), m, k).cpu().numpy().reshape(ref.shape)
    recall, gap = _recall_check(got, ref, scores, nvis, k)
    say(f"  recall {recall:.5f} worst relative gap of a swapped entry {gap:.2e}")
    assert recall >= 0.995 and gap <= 1e-3
    short = got[-1]
    assert np.array_equal(short[: k // 2], np.arange(k // 2)) and (short[k // 2:] == -1).all()


# ------------------------------------------------------------------ kv_prepare

@pytest.mark.parametrize("dtype,D,r,m,off,j0,n,gamma,inplace", [
    ("bf16", 512, 64, 4, 0, 0, None, False, True), ("bf16", 512, 64, 128, 37, 100, 300, True, False),
    ("f32", 128, 64, 4, 5, 3, 17, True, True), ("bf16", 64, 16, 1, 0, 0, None, True, False),
    ("bf16", 4096, 64, 4, 0, 7, 9, False, True)])
def test_kv_prepare(dtype, D, r, m, off, j0, n, gamma, inplace):
    say(f"kv_prepare {dtype} D={D} r={r} m={m} off={off} j0={j0} n={n} gamma={gamma} inplace={inplace}")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    g = torch.Generator().manual_seed(D + r + m)
    B, N = 3, 1200 if D < 4096 else 40
    x = (torch.randn(B, N, D, generator=g) * 3).to(tdt)
    gk = torch.rand(D, generator=g) + 0.5 if gamma else None
    kw = dict(m=m, rope_dims=r, rope_base=10000.0, entry_pos_offset=off, gamma_kv=gk, j0=j0, n=n)
    ref = oracle.kv_prepare(x, **kw)
    xd = _d(x)
    kwd = dict(kw, gamma_kv=None if gk is None else _d(gk))
    out = torch.full_like(xd, 7.0) if not inplace else None
    got = cakv.kv_prepare(xd, out=out, **kwd)
    nn = N - j0 if n is None else n
    got_c = got.float().cpu().numpy()
    # entries outside [j0, j0+n) are untouched
    other = np.ones(N, bool)
    other[j0:j0 + nn] = False
    want_other = x.float().numpy() if inplace else np.full((B, N, D), 7.0)
    assert np.array_equal(got_c[:, other], want_other[:, other])
    got_c = got_c[:, j0:j0 + nn]
    scale = np.abs(ref).max(axis=-1, keepdims=True)
    if dtype == "f32":
        assert np.all(np.abs(got_c - ref) <= 2e-6 * scale)
    else:
        assert np.all(np.abs(got_c - ref) <= _bf16_ulp(ref) + 1e-6 * scale)


# ------------------------------------------------------------------ attention

def _prep(kv, m, kw):
    """The compressed cache as the attention calls read it: a device copy with
    every entry prepared by kv_prepare."""
    return cakv.kv_prepare(_d(kv).clone(), m=m, rope_dims=kw["rope_dims"], rope_base=kw.get("rope_base", 10000.0))


def _prep_raw(raw, raw_pos0, kw):
    """The window rows as the attention calls read them: a device copy with row r
    of sequence b prepared at position raw_pos0[b] + r."""
    return cakv.kv_prepare_raw(_d(raw).clone(), np.asarray(raw_pos0).tolist(), rope_dims=kw["rope_dims"],
                               rope_base=kw.get("rope_base", 10000.0))


def _attn_check(out, ref, what):
    out = out.astype(np.float64)
    err = np.abs(out - ref)
    rel_rms = np.linalg.norm(out - ref) / np.linalg.norm(ref)
    worst = np.unravel_index(np.argmax(err), err.shape)
    say(f"  {what}: max-abs {err.max():.3e} rel-RMS {rel_rms:.3e} worst at {worst}")
    assert np.all(np.isfinite(out))
    assert err.max() <= 2e-2 and rel_rms <= 5e-3


def _attn_kw(w):
    return dict(m=w.m, n_win=w.n_win, rope_dims=w.rope_dims, rope_base=w.rope_base)


def test_sparse_attention_tiny_layer_f32():
    say("sparse attention tiny layer f32")
    inp, w, keys = _indexer_inputs("tiny_csa_f32")
    kvc = oracle.kv_compress(inp["kv"], inp["gate"], w.m).astype(np.float32)
    idx = oracle.indexer_topk(inp["q_idx"], inp["w"], inp["q_pos"], w.m, w.k,
                              k_f32=keys.astype(np.float32)).reshape(1, w.Q, w.k)
    kw = _attn_kw(w)
    ref, lse_ref = oracle.attention(inp["q"], kvc, inp["kv_raw"], inp["raw_pos0"], inp["q_pos"], inp["sinks"],
                                    idx=idx, **kw)
    for odt in (torch.float32, torch.bfloat16):
        out, lse = cakv.sparse_mqa_fwd(_d(inp["q"]), _prep(kvc, w.m, kw), _d(idx),
                                       _prep_raw(inp["kv_raw"], inp["raw_pos0"], kw),
                                       _d(inp["raw_pos0"]), _d(inp["q_pos"]), _d(inp["sinks"]), out_dtype=odt, **kw)
        _attn_check(out.float().cpu().numpy().reshape(ref.shape), ref, f"out {odt}")
    assert np.abs(lse.cpu().numpy().reshape(lse_ref.shape) - lse_ref).max() < 1e-3


def test_dense_attention_tiny_hca_f32():
    say("dense attention tiny HCA (m=128) f32")
    inp = make_inputs("tiny_csa_f32")
    w = inp["workload"].replace(m=128)
    kvc = oracle.kv_compress(inp["kv"], inp["gate"], 128).astype(np.float32)
    kw = _attn_kw(w)
    ref, lse_ref = oracle.attention(inp["q"], kvc, inp["kv_raw"], inp["raw_pos0"], inp["q_pos"], inp["sinks"], **kw)
    out, lse = cakv.dense_compressed_mqa_fwd(_d(inp["q"]), _prep(kvc, 128, kw),
                                             _prep_raw(inp["kv_raw"], inp["raw_pos0"], kw),
                                             _d(inp["raw_pos0"]), _d(inp["q_pos"]), _d(inp["sinks"]),
                                             out_dtype=torch.float32, **kw)
    _attn_check(out.cpu().numpy().reshape(ref.shape), ref, "out")
    assert np.abs(lse.cpu().numpy().reshape(lse_ref.shape) - lse_ref).max() < 1e-3


def test_sparse_attention_csa_decode_128k():
    say("sparse attention CSA decode 128K (32 queries, oracle indices)")
    inp, w, keys = _indexer_inputs("csa_decode_128k")
    codes, scale = oracle.q8_quantize(keys)
    idx = oracle.indexer_topk(inp["q_idx"], inp["w"], inp["q_pos"], w.m, w.k, k_code=codes, k_scale=scale)
    idx = idx.reshape(w.B, w.Q, w.k)
    kw = _attn_kw(w)
    ref, lse_ref = oracle.attention(inp["q"], inp["kv"], inp["kv_raw"], inp["raw_pos0"], inp["q_pos"], inp["sinks"],
                                    idx=idx, **kw)
    out, lse = cakv.sparse_mqa_fwd(_d(inp["q"]), _prep(inp["kv"], w.m, kw), _d(idx),
                                   _prep_raw(inp["kv_raw"], inp["raw_pos0"], kw),
                                   _d(inp["raw_pos0"]), _d(inp["q_pos"]), _d(inp["sinks"]), **kw)
    _attn_check(out.float().cpu().numpy().reshape(ref.shape), ref, "out bf16")
    assert np.abs(lse.cpu().numpy().reshape(lse_ref.shape) - lse_ref).max() < 1e-2


def test_dense_attention_hca_decode_1m():
    say("dense attention HCA decode 1M (32 queries x 8192 entries)")
    inp = make_inputs("hca_decode_1m")
    w = inp["workload"]
    kw = _attn_kw(w)
    ref, lse_ref = oracle.attention(inp["q"], inp["kv"], inp["kv_raw"], inp["raw_pos0"], inp["q_pos"], inp["sinks"],
                                    **kw)
    out, lse = cakv.dense_compressed_mqa_fwd(_d(inp["q"]), _prep(inp["kv"], w.m, kw),
                                             _prep_raw(inp["kv_raw"], inp["raw_pos0"], kw),
                                             _d(inp["raw_pos0"]), _d(inp["q_pos"]), _d(inp["sinks"]), **kw)
    _attn_check(out.float().cpu().numpy().reshape(ref.shape), ref, "out bf16")
    assert np.abs(lse.cpu().numpy().reshape(lse_ref.shape) - lse_ref).max() < 1e-2


def _prefill_rows(Q, n=64):
    """64 chunk rows: the first and last rows, rows on either side of m = 4
    and 128-token block boundaries (the chunk starts on one), and seeded
    random rows to fill the count."""
    fixed = list(range(8)) + [126, 127, 128, 129, 130, 131]
    for b in (256, 512, 1024, 2048, 3072, 4096, 5120, 6144, 7168):
        fixed += [b - 1, b, b + 1]
    fixed += [8060] + list(range(Q - 8, Q))
    fixed = sorted(set(r for r in fixed if r < Q))
    rng = np.random.default_rng(64)
    rest = [r for r in rng.permutation(Q).tolist() if r not in fixed][: n - len(fixed)]
    return np.array(sorted(fixed + rest), dtype=np.int64)


def test_prefill_chunk_256k_sampled_rows():
    """The CSA + HCA chunked prefill at full size (8192 query tokens after a
    262,144-token prefix) in the launch configuration the benchmark times;
    sampled rows (chunk ends and m / 128-token block boundaries) are checked
    against the oracle: the compressed caches, the selection (fp8 recall) and
    both attention layers, each fed the same inputs on both sides."""
    say("prefill chunk 256K: inputs")
    inp = make_inputs("prefill_chunk_256k")
    w = inp["workload"]
    T, Q = w.T, w.Q
    rows = _prefill_rows(Q)
    sel = torch.from_numpy(rows)
    kw = _attn_kw(w)

    # S1 at full size: GPU compression of every raw token against the oracle's
    say("  kv_compress: CSA (m=4), HCA (m=128), indexer keys (m=4, fp8)")
    kv_d = _d(inp["kv"])
    for gate, mm in ((inp["gate"], w.m), (inp["hca_gate"], w.m_hca)):
        got = cakv.kv_compress(kv_d, _d(gate), mm).float().cpu()
        ent = torch.tensor([0, 1, T // mm // 2, T // mm - 2, T // mm - 1])
        ref = oracle.kv_compress(inp["kv"][:, : T // mm * mm].view(1, T // mm, mm, -1)[:, ent].reshape(1, -1, w.D),
                                 gate[:, : T // mm * mm].view(1, T // mm, mm)[:, ent].reshape(1, -1), mm)
        diff = np.abs(got[:, ent].numpy() - ref)
        xs = inp["kv"][:, : T // mm * mm].view(1, T // mm, mm, -1)[:, ent].reshape(1, -1, w.D)
        gs = gate[:, : T // mm * mm].view(1, T // mm, mm)[:, ent].reshape(1, -1)
        assert np.all(diff <= _compress_bound(xs, gs, mm, ref, True)), diff.max()

    # caches from the oracle, fed to both sides from here on
    kvc = torch.from_numpy(oracle.kv_compress(inp["kv"], inp["gate"], w.m)).to(torch.bfloat16)
    kvh = torch.from_numpy(oracle.kv_compress(inp["kv"], inp["hca_gate"], w.m_hca)).to(torch.bfloat16)
    keys = oracle.kv_compress(inp["k_idx"], inp["k_gate"], w.m)
    codes, scale = oracle.q8_quantize(keys)

    say("  indexer top-k, 8192 queries x 67,584 entries")
    idx = cakv.indexer_topk(_d(inp["q_idx"]), _d(inp["w"]), _d(codes), _d(scale), _d(inp["q_pos"]), w.m, w.k)
    idx_rows = idx[:, sel].cpu().numpy()
    scores, nvis = oracle.indexer_scores(inp["q_idx"][:, sel], inp["w"][:, sel], inp["q_pos"][:, sel], w.m,
                                         k_code=codes, k_scale=scale)
    ref = oracle.topk(scores, nvis, w.k)
    recall, gap = _recall_check(idx_rows.reshape(ref.shape), ref, scores, nvis, w.k)
    say(f"  recall {recall:.5f} worst relative gap of a swapped entry {gap:.2e}")
    assert recall >= 0.995 and gap <= 1e-3

    say("  CSA layer: sparse attention over the selection + window + sinks")
    win = _prep_raw(inp["kv"], inp["raw_pos0"], kw)
    out, _ = cakv.sparse_mqa_fwd(_d(inp["q"]), _prep(kvc, w.m, kw), idx, win, _d(inp["raw_pos0"]),
                                 _d(inp["q_pos"]), _d(inp["sinks"]), want_lse=False, **kw)
    ref, _ = oracle.attention(inp["q"][:, sel], kvc, inp["kv_raw"], inp["raw_pos0"], inp["q_pos"][:, sel],
                              inp["sinks"], idx=idx_rows, **kw)
    _attn_check(out[:, sel].float().cpu().numpy().reshape(ref.shape), ref, "CSA out")

    say("  HCA layer: dense attention over every visible entry + window + sinks")
    kwh = dict(kw, m=w.m_hca)
    out, _ = cakv.dense_compressed_mqa_fwd(_d(inp["q_hca"]), _prep(kvh, w.m_hca, kw), win, _d(inp["raw_pos0"]),
                                           _d(inp["q_pos"]), _d(inp["sinks_hca"]), want_lse=False, **kwh)
    ref, _ = oracle.attention(inp["q_hca"][:, sel], kvh, inp["kv_raw"], inp["raw_pos0"], inp["q_pos"][:, sel],
                              inp["sinks_hca"], **kwh)
    _attn_check(out[:, sel].float().cpu().numpy().reshape(ref.shape), ref, "HCA out")


def test_attention_edge_cases():
    """Early rows (t < m: window and sink only), an empty key set with a -inf
    sink, K = 0 slots, duplicate-free padding, positions outside the raw rows."""
    say("attention edge cases")
    g = torch.Generator().manual_seed(5)
    B, Q, H, D, N, R, K = 2, 6, 128, 512, 40, 8, 16
    q = torch.randn(B, Q, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    raw = torch.randn(B, R, D, generator=g).to(torch.bfloat16)
    sinks = torch.randn(H, generator=g)
    sinks[3] = -math.inf
    qpos = torch.tensor([[0, 1, 3, 5, 100, 1000], [2, 7, 60, 61, 159, 163]], dtype=torch.int32)
    raw0 = torch.tensor([0, 156], dtype=torch.int32)  # sequence 1: raw rows cover positions 156..163 only
    idx = torch.randint(0, N, (B, Q, K), generator=g, dtype=torch.int32)
    for b in range(B):
        for i in range(Q):
            idx[b, i] = torch.randperm(N, generator=g)[:K].to(torch.int32)
    idx[:, :, ::3] = -1
    kw = dict(m=4, n_win=4, rope_dims=64)
    ref, lse_ref = oracle.attention(q, kv, raw, raw0, qpos, sinks, idx=idx.numpy(), **kw)
    kvp, rawp = _prep(kv, 4, kw), _prep_raw(raw, raw0, kw)
    out, lse = cakv.sparse_mqa_fwd(_d(q), kvp, _d(idx), rawp, _d(raw0), _d(qpos), _d(sinks),
                                   out_dtype=torch.float32, **kw)
    _attn_check(out.cpu().numpy().reshape(ref.shape), ref, "sparse edge")
    lg = lse.cpu().numpy().reshape(lse_ref.shape)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lg), fin) and np.abs(lg[fin] - lse_ref[fin]).max() < 1e-2  # bf16 logits
    ref2, _ = oracle.attention(q, kv, raw, raw0, qpos, sinks, **kw)
    out2, _ = cakv.dense_compressed_mqa_fwd(_d(q), kvp, rawp, _d(raw0), _d(qpos), _d(sinks),
                                            out_dtype=torch.float32, **kw)
    _attn_check(out2.cpu().numpy().reshape(ref2.shape), ref2, "dense edge")
    # no window, no entries, -inf sinks: zero output, lse -inf
    sk = torch.full((H,), -math.inf)
    out3, lse3 = cakv.dense_compressed_mqa_fwd(_d(q), kvp[:, :0], rawp, _d(raw0), _d(qpos), _d(sk),
                                               out_dtype=torch.float32, m=4, n_win=0, rope_dims=64)
    assert torch.all(out3 == 0) and torch.all(torch.isneginf(lse3))


def test_attention_split_combine_odd_heads():
    """Several key splits merged by the combine kernel: an odd head count (the
    last head pair holds one head), a -inf sink and the lse."""
    say("attention split combine, odd head count")
    g = torch.Generator().manual_seed(11)
    B, Q, H, D, N, R = 3, 1, 5, 128, 2000, 64
    q = torch.randn(B, Q, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    raw = torch.randn(B, R, D, generator=g).to(torch.bfloat16)
    sinks = torch.randn(H, generator=g)
    sinks[2] = -math.inf
    qpos = torch.tensor([[4 * N + 10], [4 * N + 30], [3000]], dtype=torch.int32)
    raw0 = (qpos[:, 0] - R + 1).to(torch.int32)
    kw = dict(m=4, n_win=16, rope_dims=32)
    ref, lse_ref = oracle.attention(q, kv, raw, raw0, qpos, sinks, **kw)
    kvp, rawp = _prep(kv, 4, kw), _prep_raw(raw, raw0, kw)
    out, lse = cakv.dense_compressed_mqa_fwd(_d(q), kvp, rawp, _d(raw0), _d(qpos), _d(sinks),
                                             out_dtype=torch.float32, **kw)
    _attn_check(out.cpu().numpy().reshape(ref.shape), ref, "split combine")
    lg = lse.cpu().numpy().reshape(lse_ref.shape)
    assert np.all(np.isfinite(lg)) and np.abs(lg - lse_ref).max() < 1e-2  # bf16 logits


def test_attention_needle_forces_exact_max_pass():
    """A key equal to the query (logit sqrt(D), far above the rest) sitting in a
    late tile: the kernel's reference max from the first tiles is too small,
    so it must take its exact-max second pass."""
    say("attention needle (second pass)")
    g = torch.Generator().manual_seed(7)
    B, Q, H, D, N = 2, 1, 128, 512, 2048
    q = torch.randn(B, Q, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    kv[0, 1900] = q[0, 0, 5]
    kv[1, 1500] = q[1, 0, 77]
    raw = torch.randn(B, 128, D, generator=g).to(torch.bfloat16)
    t = 4 * N
    qpos = torch.full((B, Q), t, dtype=torch.int32)
    raw0 = torch.full((B,), t - 127, dtype=torch.int32)
    sinks = torch.randn(H, generator=g)
    kw = dict(m=4, n_win=128, rope_dims=0)
    ref, _ = oracle.attention(q, kv, raw, raw0, qpos, sinks, **kw)
    out, _ = cakv.dense_compressed_mqa_fwd(_d(q), _prep(kv, 4, kw), _prep_raw(raw, raw0, kw), _d(raw0), _d(qpos),
                                           _d(sinks),
                                           out_dtype=torch.float32, **kw)
    _attn_check(out.cpu().numpy().reshape(ref.shape), ref, "needle")
    assert np.abs(ref[0, 5]).max() > 0.5  # the needle dominates that head


def test_determinism():
    say("determinism")
    inp = make_inputs("csa_decode_128k", B=4)
    w = inp["workload"]
    idx = torch.randint(0, w.N, (w.B, w.Q, w.k), dtype=torch.int32)
    args = (_d(inp["q"]), _prep(inp["kv"], w.m, _attn_kw(w)), _d(idx),
            _prep_raw(inp["kv_raw"], inp["raw_pos0"], _attn_kw(w)), _d(inp["raw_pos0"]),
            _d(inp["q_pos"]), _d(inp["sinks"]))
    a, la = cakv.sparse_mqa_fwd(*args, **_attn_kw(w))
    b, lb = cakv.sparse_mqa_fwd(*args, **_attn_kw(w))
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_sparse_attention_csa_decode_1m():
    """CSA decode at 1M context at full size and in the launch configuration
    the benchmark times (8 queries, 262,144 entries each, k = 1024 + a
    128-token window: nine key splits merged by the combine kernel), fed the
    oracle's fp8-mode indices."""
    say("sparse attention CSA decode 1M (8 queries x 262,144 entries, oracle indices)")
    inp, w, keys = _indexer_inputs("csa_decode_1m")
    codes, scale = oracle.q8_quantize(keys)
    del keys
    idx = oracle.indexer_topk(inp["q_idx"], inp["w"], inp["q_pos"], w.m, w.k, k_code=codes, k_scale=scale)
    idx = idx.reshape(w.B, w.Q, w.k)
    assert np.all(idx >= 0)  # 262,144 visible entries: every slot is filled
    kw = _attn_kw(w)
    assert cakv.sparse_mqa_workspace_bytes(w.B, w.Q, w.H, w.D, w.k, w.n_win) > 0  # several splits
    ref, lse_ref = oracle.attention(inp["q"], inp["kv"], inp["kv_raw"], inp["raw_pos0"], inp["q_pos"], inp["sinks"],
                                    idx=idx, **kw)
    out, lse = cakv.sparse_mqa_fwd(_d(inp["q"]), _prep(inp["kv"], w.m, kw), _d(idx),
                                   _prep_raw(inp["kv_raw"], inp["raw_pos0"], kw),
                                   _d(inp["raw_pos0"]), _d(inp["q_pos"]), _d(inp["sinks"]), **kw)
    _attn_check(out.float().cpu().numpy().reshape(ref.shape), ref, "out bf16")
    assert np.abs(lse.cpu().numpy().reshape(lse_ref.shape) - lse_ref).max() < 1e-2


@pytest.mark.parametrize("case", ["bf16_one_split", "bf16_splits", "f32"])
def test_attention_learned_scales(case):
    """The learned half of QK-RMSNorm and the call's scalar parameters on the
    GPU: random gamma_q and gamma_kv, softmax_scale 0.05, rms_eps 1e-5 and a
    compressed-entry position offset of 3, for bf16 D = 512 with one split per
    query (256 queries: the forward kernel's own epilogue) and with several
    (4 queries: split partials and the combine), and for f32 D = 128.  The GPU
    prepares its rows with the same gamma_kv, eps and offset; the oracle
    attends over the raw rows with the same parameters."""
    say(f"attention with gamma_q, gamma_kv, softmax_scale, rms_eps, entry offset: {case}")
    g = torch.Generator().manual_seed({"bf16_one_split": 21, "bf16_splits": 22, "f32": 23}[case])
    if case == "f32":
        B, Q, H, D, N, R, K, r, dt = 2, 8, 8, 128, 500, 16, 64, 32, torch.float32
    elif case == "bf16_one_split":
        B, Q, H, D, N, R, K, r, dt = 2, 128, 128, 512, 300, 32, 64, 64, torch.bfloat16
    else:
        B, Q, H, D, N, R, K, r, dt = 4, 1, 128, 512, 3000, 128, 1024, 64, torch.bfloat16
    m, n_win, off, eps, tau = 4, min(R, 32), 3, 1e-5, 0.05
    q = torch.randn(B, Q, H, D, generator=g).to(dt)
    kv = (torch.randn(B, N, D, generator=g) * 2).to(dt)
    raw = torch.randn(B, R, D, generator=g).to(dt)
    sinks = torch.randn(H, generator=g)
    gq = torch.rand(D, generator=g) + 0.5
    gk = torch.rand(D, generator=g) + 0.5
    qpos = torch.randint(4 * N - 50, 4 * N + 40, (B, Q), generator=g, dtype=torch.int32)
    qpos[0, 0] = 2  # an early row: window and sink only
    raw0 = (qpos.max(dim=1).values - R + 1).clamp(min=0).to(torch.int32)
    idx = torch.stack([torch.stack([torch.randperm(N, generator=g)[:K] for _ in range(Q)]) for _ in range(B)])
    idx = idx.sort(dim=-1).values.to(torch.int32)
    idx[:, :, ::7] = -1
    kw = dict(m=m, n_win=n_win, rope_dims=r, rope_base=10000.0, softmax_scale=tau, rms_eps=eps)
    kvp = cakv.kv_prepare(_d(kv).clone(), m=m, rope_dims=r, entry_pos_offset=off, rms_eps=eps, gamma_kv=_d(gk))
    rawp = cakv.kv_prepare_raw(_d(raw).clone(), raw0.tolist(), rope_dims=r, rms_eps=eps, gamma_kv=_d(gk))
    # (the split count follows the batch: 256 queries fill the GPU with one
    # split each, 4 queries of 1,056 key slots take 8 splits)
    ref, lse_ref = oracle.attention(q, kv, raw, raw0, qpos, sinks, idx=idx.numpy(), entry_pos_offset=off,
                                    gamma_q=gq, gamma_kv=gk, **kw)
    out, lse = cakv.sparse_mqa_fwd(_d(q), kvp, _d(idx), rawp, _d(raw0), _d(qpos), _d(sinks), gamma_q=_d(gq),
                                   out_dtype=torch.float32, **kw)
    _attn_check(out.cpu().numpy().reshape(ref.shape), ref, f"sparse {case}")
    assert np.abs(lse.cpu().numpy().reshape(lse_ref.shape) - lse_ref).max() < 1e-2
    ref2, _ = oracle.attention(q, kv, raw, raw0, qpos, sinks, entry_pos_offset=off, gamma_q=gq, gamma_kv=gk, **kw)
    out2, _ = cakv.dense_compressed_mqa_fwd(_d(q), kvp, rawp, _d(raw0), _d(qpos), _d(sinks), gamma_q=_d(gq),
                                            out_dtype=torch.bfloat16, **kw)
    _attn_check(out2.float().cpu().numpy().reshape(ref2.shape), ref2, f"dense {case}")


def _poison(t, byte):
    t.view(torch.uint8).fill_(byte)
    return t


def test_outputs_and_workspaces_are_fully_overwritten():
    """Outputs pre-filled with poison bytes (0xFF: NaN in every float type;
    0x5A5A5A5A, an index out of range, for idx) are fully overwritten, and a
    workspace full of 0xFF gives bitwise the same results as a zeroed one:
    no call reads anything it did not write first."""
    say("poisoned outputs and workspaces")
    inp = make_inputs("csa_decode_128k", B=2)
    w = inp["workload"]
    codes, scale = oracle.q8_quantize(inp["k_idx"].numpy())
    nws = cakv.indexer_topk_workspace_bytes(w.B, w.Q, w.N, w.k)
    results = []
    for byte in (0x00, 0xFF):
        ws = _poison(torch.empty(nws, dtype=torch.uint8, device=DEV), byte)
        out = _poison(torch.empty((w.B, w.Q, w.k), dtype=torch.int32, device=DEV), 0x5A)
        results.append(cakv.indexer_topk(_d(inp["q_idx"]), _d(inp["w"]), _d(codes), _d(scale), _d(inp["q_pos"]),
                                         w.m, w.k, out=out, workspace=ws).cpu())
    assert torch.equal(results[0], results[1])
    assert bool(((results[0] >= 0) & (results[0] < w.N)).all())
    idx = results[0].to(DEV)

    kw = _attn_kw(w)
    kvp, rawp = _prep(inp["kv"], w.m, kw), _prep_raw(inp["kv_raw"], inp["raw_pos0"], kw)
    args = (_d(inp["q"]), kvp, idx, rawp, _d(inp["raw_pos0"]), _d(inp["q_pos"]), _d(inp["sinks"]))
    nwa = cakv.sparse_mqa_workspace_bytes(w.B, w.Q, w.H, w.D, w.k, w.n_win)
    assert nwa > 0  # two queries: split partials
    outs = []
    for byte in (0x00, 0xFF):
        ws = _poison(torch.empty(nwa, dtype=torch.uint8, device=DEV), byte)
        o = _poison(torch.empty((w.B, w.Q, w.H, w.D), dtype=torch.bfloat16, device=DEV), 0xFF)
        o, l = cakv.sparse_mqa_fwd(*args, out=o, workspace=ws, **kw)
        outs.append((o.cpu(), l.cpu()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    assert bool(torch.isfinite(outs[0][0].float()).all()) and bool(torch.isfinite(outs[0][1]).all())

    # one split per query (256 queries): the forward kernel writes the output itself
    g = torch.Generator().manual_seed(3)
    q = torch.randn(1, 256, 128, 512, generator=g).to(torch.bfloat16)
    kv = torch.randn(1, 200, 512, generator=g).to(torch.bfloat16)
    raw = torch.randn(1, 300, 512, generator=g).to(torch.bfloat16)
    qpos = torch.arange(44, 300, dtype=torch.int32).view(1, 256)
    raw0 = torch.zeros(1, dtype=torch.int32)
    kwd = dict(m=4, n_win=16, rope_dims=64)
    kvd, rawd = _prep(kv, 4, kwd), _prep_raw(raw, raw0, kwd)
    o = _poison(torch.empty((1, 256, 128, 512), dtype=torch.bfloat16, device=DEV), 0xFF)
    o, l = cakv.dense_compressed_mqa_fwd(_d(q), kvd, rawd, _d(raw0), _d(qpos), _d(inp["sinks"]), out=o, **kwd)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(l).all())
    ref, _ = oracle.attention(q, kv, raw, raw0, qpos, inp["sinks"], **kwd)
    _attn_check(o.float().cpu().numpy().reshape(ref.shape), ref, "one-split dense")

    # kv_compress: every output byte and scale written
    for odt in (torch.bfloat16, torch.float8_e4m3fn):
        x = torch.randn(2, 1030, 128, generator=g).to(torch.bfloat16)
        gate = torch.randn(2, 1030, generator=g)
        o = _poison(torch.empty((2, 1030 // 4, 128), dtype=odt, device=DEV), 0xFF)
        sc = _poison(torch.empty((2, 1030 // 4), dtype=torch.float32, device=DEV), 0xFF) \
            if odt == torch.float8_e4m3fn else None
        res = cakv.kv_compress(_d(x), _d(gate), 4, out=o, scale=sc)
        fresh = cakv.kv_compress(_d(x), _d(gate), 4, odt)
        if odt == torch.float8_e4m3fn:
            assert torch.equal(res[0].view(torch.uint8), fresh[0].view(torch.uint8))
            assert torch.equal(res[1], fresh[1])
        else:
            assert torch.equal(res.view(torch.uint16), fresh.view(torch.uint16))
