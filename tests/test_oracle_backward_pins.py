"""Pins of the oracle's backward functions (training), CPU only.

Each gradient is checked against
  * torch autograd in fp64 over an explicit formula written here from the
    pages' definitions (independent of the oracle's hand-written chain rule),
  * central finite differences of the oracle's own forward functions, which
    test_oracle_pins.py pins against the pages and textbook routines,
  * closed forms (a single key: the query gets no gradient; all terms
    non-negative: the absolute sums equal the signed ones).
"""
import math

import numpy as np
import pytest
import torch

import oracle



@pytest.fixture(autouse=True)
def _fp64_default():
    """fp64 tensors by default inside these tests only (restored afterwards, so
    other test modules collected in the same process keep torch's default)"""
    prev = torch.get_default_dtype()
    torch.set_default_dtype(torch.float64)
    yield
    torch.set_default_dtype(prev)


def _rope_t(x, pos, r, base=10000.0):
    """rotate the trailing r dims of x [..., D] by pos [...] (consecutive pairs)"""
    if r == 0:
        return x
    D = x.shape[-1]
    i = torch.arange(r // 2, dtype=torch.float64)
    ang = pos[..., None].double() * base ** (-2.0 * i / r)
    c, s = torch.cos(ang), torch.sin(ang)
    a, b = x[..., D - r::2], x[..., D - r + 1::2]
    ra, rb = a * c - b * s, a * s + b * c
    rot = torch.stack([ra, rb], dim=-1).reshape(*x.shape[:-1], r)
    return torch.cat([x[..., :D - r], rot], dim=-1)


def _rms_t(x, gamma, eps):
    y = x / torch.sqrt((x * x).mean(dim=-1, keepdim=True) + eps)
    return y if gamma is None else y * gamma


def _case(seed, B=2, Q=3, H=4, D=16, N=12, R=10, K=5, r=8, sparse=True):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Q, H, D, generator=g, dtype=torch.float32)
    kv = torch.randn(B, N, D, generator=g, dtype=torch.float32) * 2
    raw = torch.randn(B, R, D, generator=g, dtype=torch.float32)
    sinks = torch.randn(H, generator=g, dtype=torch.float32)
    gq = torch.rand(D, generator=g, dtype=torch.float32) + 0.5
    gk = torch.rand(D, generator=g, dtype=torch.float32) + 0.5
    qpos = torch.randint(4, 4 * N + 6, (B, Q), generator=g, dtype=torch.int32)
    raw0 = (qpos.max(dim=1).values - R + 1).clamp(min=0).to(torch.int32)
    idx = None
    if sparse:
        idx = torch.stack([torch.stack([torch.randperm(N, generator=g)[:K] for _ in range(Q)]) for _ in range(B)])
        idx = idx.to(torch.int32)
        idx[:, :, 1] = -1
    dout = torch.randn(B, Q, H, D, generator=g, dtype=torch.float32)
    kw = dict(m=4, n_win=6, rope_dims=r, rope_base=10000.0, entry_pos_offset=1, softmax_scale=0.3, rms_eps=1e-5)
    return dict(q=q, kv=kv, raw=raw, sinks=sinks, gq=gq, gk=gk, qpos=qpos, raw0=raw0, idx=idx, dout=dout, kw=kw)


def _attn_torch(c, khat_c, khat_raw, q, sinks, gq):
    """sum(dout * out) of the attention, from the definitions: one softmax over
    the selected (or all visible) compressed entries, the raw window and the
    sink; keys = values = the prepared rows (leaf tensors here)."""
    kw = c["kw"]
    B, Q, H, D = q.shape
    N, R = khat_c.shape[1], khat_raw.shape[1]
    tau = kw["softmax_scale"]
    loss = 0.0
    for b in range(B):
        for i in range(Q):
            t = int(c["qpos"][b, i])
            nv = min(t // kw["m"], N)
            rows = []
            ents = c["idx"][b, i].tolist() if c["idx"] is not None else list(range(nv))
            for j in ents:
                if 0 <= j < nv:
                    rows.append(khat_c[b, j])
            for p in range(max(0, t - kw["n_win"] + 1), t + 1):
                rr = p - int(c["raw0"][b])
                if 0 <= rr < R:
                    rows.append(khat_raw[b, rr])
            keys = torch.stack(rows) if rows else torch.zeros(0, D)
            qh = _rope_t(_rms_t(q[b, i].double(), gq, kw["rms_eps"]), torch.tensor([t] * H), kw["rope_dims"])
            logits = tau * qh @ keys.T  # [H, n]
            allz = torch.cat([logits, sinks.double()[:, None]], dim=1)
            p = torch.softmax(allz, dim=1)[:, :-1]
            o = p @ keys
            out = _rope_t(o, torch.tensor([-t] * H), kw["rope_dims"])
            loss = loss + (c["dout"][b, i].double() * out).sum()
    return loss


def _prepared(c):
    kw = c["kw"]
    kc = oracle.kv_prepare(c["kv"], m=kw["m"], rope_dims=kw["rope_dims"], entry_pos_offset=kw["entry_pos_offset"],
                           rms_eps=kw["rms_eps"], gamma_kv=c["gk"])
    B, R = c["raw"].shape[:2]
    kr = np.concatenate([oracle.kv_prepare(c["raw"][b:b + 1], m=1, rope_dims=kw["rope_dims"],
                                           entry_pos_offset=int(c["raw0"][b]), rms_eps=kw["rms_eps"],
                                           gamma_kv=c["gk"]) for b in range(B)])
    return torch.from_numpy(kc), torch.from_numpy(kr)


@pytest.mark.parametrize("sparse", [True, False])
def test_attention_bwd_matches_autograd(sparse):
    c = _case(1 if sparse else 2, sparse=sparse)
    got = oracle.attention_bwd(c["q"], c["kv"], c["raw"], c["raw0"], c["qpos"], c["sinks"], c["dout"], idx=c["idx"],
                               gamma_q=c["gq"], gamma_kv=c["gk"], **c["kw"])
    khat_c, khat_raw = _prepared(c)
    khat_c.requires_grad_(True)
    khat_raw.requires_grad_(True)
    q = c["q"].double().requires_grad_(True)
    sinks = c["sinks"].double().requires_grad_(True)
    gq = c["gq"].double().requires_grad_(True)
    _attn_torch(c, khat_c, khat_raw, q, sinks, gq).backward()
    for name, ref in (("dq", q.grad), ("dkhat_c", khat_c.grad), ("dkhat_raw", khat_raw.grad),
                      ("dsinks", sinks.grad), ("dgamma_q", gq.grad)):
        assert np.allclose(got[name], ref.numpy(), rtol=1e-9, atol=1e-11), name
    assert np.abs(got["dkhat_raw"]).max() > 0 and np.abs(got["dkhat_c"]).max() > 0


def test_attention_bwd_finite_differences():
    """Central differences of sum(dout * out) from the forward oracle, for
    query elements, raw cache and window elements (through kv_prepare's
    gradient) and sink logits."""
    c = _case(3)
    kw = c["kw"]
    got = oracle.attention_bwd(c["q"], c["kv"], c["raw"], c["raw0"], c["qpos"], c["sinks"], c["dout"], idx=c["idx"],
                               gamma_q=c["gq"], gamma_kv=c["gk"], **kw)
    dkv, _ = oracle.kv_prepare_bwd(c["kv"], got["dkhat_c"], m=kw["m"], rope_dims=kw["rope_dims"],
                                   entry_pos_offset=kw["entry_pos_offset"], rms_eps=kw["rms_eps"], gamma_kv=c["gk"])

    def loss(q=None, kv=None, raw=None, sinks=None):
        o, _ = oracle.attention(c["q"] if q is None else q, c["kv"] if kv is None else kv,
                                c["raw"] if raw is None else raw, c["raw0"], c["qpos"],
                                c["sinks"] if sinks is None else sinks, idx=c["idx"], gamma_q=c["gq"],
                                gamma_kv=c["gk"], **kw)
        return float((o.reshape(c["dout"].shape) * c["dout"].double().numpy()).sum())

    h = 2.0 ** -12
    rng = np.random.default_rng(0)
    for name, arr, grad in (("q", c["q"], got["dq"]), ("kv", c["kv"], dkv), ("sinks", c["sinks"], got["dsinks"])):
        for _ in range(6):
            pos = tuple(rng.integers(0, s) for s in arr.shape)
            if name == "kv" and abs(grad[pos]) < 1e-6:
                continue
            plus, minus = arr.clone(), arr.clone()
            plus[pos] += h
            minus[pos] -= h
            fd = (loss(**{name: plus}) - loss(**{name: minus})) / (2 * h)
            assert abs(fd - grad[pos]) <= 1e-5 * max(1.0, abs(grad[pos])), (name, pos, fd, grad[pos])
    # the window rows' gradient through kv_prepare, for one sequence
    b = 1
    dr, _ = oracle.kv_prepare_bwd(c["raw"][b:b + 1], got["dkhat_raw"][b:b + 1], m=1, rope_dims=kw["rope_dims"],
                                  entry_pos_offset=int(c["raw0"][b]), rms_eps=kw["rms_eps"], gamma_kv=c["gk"])
    nz = np.argwhere(np.abs(dr[0]) > 1e-6)
    for rr, d in nz[:6]:
        plus, minus = c["raw"].clone(), c["raw"].clone()
        plus[b, rr, d] += h
        minus[b, rr, d] -= h
        fd = (loss(raw=plus) - loss(raw=minus)) / (2 * h)
        assert abs(fd - dr[0, rr, d]) <= 1e-5 * max(1.0, abs(dr[0, rr, d]))


def test_attention_bwd_single_key_closed_form():
    """One key and a -inf sink: out = RoPE_-t(k_hat) whatever the query, so
    dq = 0 and d k_hat = RoPE_t(dout)."""
    g = torch.Generator().manual_seed(4)
    D, H = 16, 3
    q = torch.randn(1, 1, H, D, generator=g, dtype=torch.float32)
    raw = torch.randn(1, 1, D, generator=g, dtype=torch.float32)
    kv = torch.zeros(1, 1, D, dtype=torch.float32)
    dout = torch.randn(1, 1, H, D, generator=g, dtype=torch.float32)
    t = 2  # m = 4: no compressed entry visible; the window is position 2 only
    qpos = torch.tensor([[t]], dtype=torch.int32)
    raw0 = torch.tensor([t], dtype=torch.int32)
    sinks = torch.full((H,), -math.inf, dtype=torch.float32)
    got = oracle.attention_bwd(q, kv, raw, raw0, qpos, sinks, dout, m=4, n_win=1, rope_dims=8)
    assert np.abs(got["dq"]).max() < 1e-12
    want = _rope_t(dout[0, 0].double(), torch.tensor([t] * H), 8).sum(dim=0).numpy()
    assert np.allclose(got["dkhat_raw"][0, 0], want, rtol=1e-12, atol=1e-12)
    assert np.all(got["dsinks"] == 0)


@pytest.mark.parametrize("gamma", [False, True])
def test_kv_prepare_bwd_matches_autograd(gamma):
    g = torch.Generator().manual_seed(5)
    B, N, D, r, m, off, j0, n = 2, 9, 24, 8, 4, 3, 2, 5
    x = torch.randn(B, N, D, generator=g, dtype=torch.float32) * 3
    gk = (torch.rand(D, generator=g, dtype=torch.float32) + 0.5) if gamma else None
    dy = torch.randn(B, n, D, generator=g)
    dx, dg = oracle.kv_prepare_bwd(x, dy.numpy(), m=m, rope_dims=r, entry_pos_offset=off, rms_eps=1e-5,
                                   gamma_kv=gk, j0=j0, n=n)
    xl = x[:, j0:j0 + n].double().requires_grad_(True)
    gl = gk.double().requires_grad_(True) if gamma else None
    pos = (torch.arange(j0, j0 + n) * m + off).expand(B, n)
    y = _rope_t(_rms_t(xl, gl, 1e-5), pos, r)
    (y * dy).sum().backward()
    assert np.allclose(dx, xl.grad.numpy(), rtol=1e-10, atol=1e-12)
    if gamma:
        assert np.allclose(dg, gl.grad.numpy(), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("m,span,per_channel", [(4, 4, False), (4, 8, False), (4, 8, True), (3, 7, True),
                                                (128, 128, False)])
def test_kv_compress_bwd_matches_autograd_and_differences(m, span, per_channel):
    g = torch.Generator().manual_seed(10 * m + span)
    B, T, D = 2, 3 * m + 2 if m < 128 else 260, 6
    x = torch.randn(B, T, D, generator=g, dtype=torch.float32)
    gate = torch.randn((B, T, D) if per_channel else (B, T), generator=g, dtype=torch.float32)
    dc = torch.randn(B, T // m, D, generator=g)
    dx, dg = oracle.kv_compress_bwd(x, gate, m, dc.numpy(), span)
    xl, gl = x.double().requires_grad_(True), gate.double().requires_grad_(True)
    outs = []
    for j in range(T // m):
        hi = (j + 1) * m
        lo = max(0, hi - span)
        gg = gl[:, lo:hi] if per_channel else gl[:, lo:hi, None].expand(B, hi - lo, D)
        outs.append((torch.softmax(gg, dim=1) * xl[:, lo:hi]).sum(dim=1))
    (torch.stack(outs, dim=1) * dc).sum().backward()
    assert np.allclose(dx, xl.grad.numpy(), rtol=1e-11, atol=1e-13)
    assert np.allclose(dg, gl.grad.numpy(), rtol=1e-11, atol=1e-13)
    # central differences of the forward oracle for a few gate logits
    h = 2.0 ** -14
    rng = np.random.default_rng(m + span)
    for _ in range(4):
        pos = tuple(rng.integers(0, s) for s in gate.shape)
        plus, minus = gate.clone(), gate.clone()
        plus[pos] += h
        minus[pos] -= h
        fd = ((oracle.kv_compress_ex(x, plus, m, span) - oracle.kv_compress_ex(x, minus, m, span)) *
              dc.numpy()).sum() / (2 * h)
        assert abs(fd - dg[pos]) <= 1e-6 * max(1.0, abs(dg[pos]))


def _indexer_case(seed, fp8=False):
    rng = np.random.default_rng(seed)
    B, Q, HI, dI, N, K, m = 2, 3, 4, 16, 40, 7, 4
    q = rng.standard_normal((B, Q, HI, dI)).astype(np.float32)
    w = rng.standard_normal((B, Q, HI)).astype(np.float32)
    keys = rng.standard_normal((B, N, dI)).astype(np.float32)
    qpos = rng.integers(4, 4 * N + 5, size=(B, Q)).astype(np.int32)
    idx = np.stack([np.stack([rng.permutation(N)[:K] for _ in range(Q)]) for _ in range(B)]).astype(np.int32)
    idx[:, :, 2] = -1
    dS = rng.standard_normal((B, Q, K)).astype(np.float32)
    kk = dict(k_f32=keys)
    if fp8:
        codes, scale = oracle.q8_quantize(keys)
        kk = dict(k_code=codes, k_scale=scale)
        keys = oracle.q8_dequantize(codes, scale)
    return q, w, keys, qpos, idx, dS, kk, m


@pytest.mark.parametrize("fp8", [False, True])
def test_indexer_bwd_matches_autograd(fp8):
    q, w, keys, qpos, idx, dS, kk, m = _indexer_case(6 + fp8, fp8)
    dq, dw, dk = oracle.indexer_bwd(q, w, qpos, m, idx, dS, **kk)
    ql, wl, kl = (torch.from_numpy(a.astype(np.float64)).requires_grad_(True) for a in (q, w, keys))
    B, Q, HI, dI = q.shape
    N = keys.shape[1]
    loss, dots = 0.0, []
    for b in range(B):
        for i in range(Q):
            nv = min(int(qpos[b, i]) // m, N)
            for s in range(idx.shape[-1]):
                j = int(idx[b, i, s])
                if 0 <= j < nv:
                    sh = ql[b, i] @ kl[b, j]
                    dots.append(sh.detach())
                    loss = loss + float(dS[b, i, s]) * (wl[b, i] * torch.relu(sh)).sum()
    loss.backward()
    assert torch.cat(dots).abs().min() > 1e-4  # no ReLU decision close to its kink
    assert np.allclose(dq, ql.grad.numpy(), rtol=1e-9, atol=1e-12)
    assert np.allclose(dw, wl.grad.numpy(), rtol=1e-9, atol=1e-12)
    assert np.allclose(dk, kl.grad.numpy(), rtol=1e-9, atol=1e-12)


def test_indexer_bwd_absolute_sums():
    q, w, keys, qpos, idx, dS, kk, m = _indexer_case(8)
    signed = oracle.indexer_bwd(q, w, qpos, m, idx, dS, **kk)
    absolute = oracle.indexer_bwd(q, w, qpos, m, idx, dS, absolute=True, **kk)
    for s_, a_ in zip(signed, absolute):
        assert np.all(a_ >= np.abs(s_) - 1e-12)
    # all terms non-negative: the two agree
    qp, wp, kp, dp = np.abs(q), np.abs(w), np.abs(keys), np.abs(dS)
    for s_, a_ in zip(oracle.indexer_bwd(qp, wp, qpos, m, idx, dp, k_f32=kp),
                      oracle.indexer_bwd(qp, wp, qpos, m, idx, dp, k_f32=kp, absolute=True)):
        assert np.allclose(s_, a_, rtol=1e-14, atol=0)
