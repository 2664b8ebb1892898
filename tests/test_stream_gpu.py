"""Parity of the compressor variants and of the streaming decode step against
the CPU oracle.

  * kv_compress_ex (spans reaching back over earlier blocks, per-channel gate
    logits): the a-priori bound of the kernel's fp32 arithmetic,
    (2n + 10) * 2^-24 * sum_i a_i |x_i| per element with n the span's token
    count (the oracle gives the sum exactly by compressing |x|), plus one
    bf16 ulp for bf16 output; fp8 within one E4M3 step of the oracle's
    dequantised value.
  * the streaming decode step (kv_append + indexer_topk + attention reading
    the window ring), token by token over more than two HCA blocks
    (2 x 128 tokens) per sequence, sequences starting at different positions:
    every step's attention outputs against the oracle run on the full prefix
    (fed the step's own selection; max-abs <= 2e-2, rel-RMS <= 5e-3), every
    step's selection against the oracle's top-k on the same dequantised keys
    (recall >= 99.5 %, misses within 1e-3 relative of the k-th score), and
    the final caches and window rings bitwise against the bulk calls
    (kv_compress_ex / kv_prepare), whose own parity the other tests check.
"""
import sys

import numpy as np
import pytest
import torch

import compressed_attention_kv_amd as cakv
import oracle

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


def _span_tokens(T, m, span):
    """tokens in each entry's span, [T//m]"""
    hi = (np.arange(T // m) + 1) * m
    return hi - np.maximum(0, hi - span)


# ------------------------------------------------------------------ compressor variants

@pytest.mark.parametrize("m,span,per_channel,odt", [
    (4, 4, True, "f32"), (4, 8, False, "bf16"), (4, 8, True, "bf16"), (4, 13, True, "f32"),
    (128, 256, False, "bf16"), (128, 128, True, "bf16"), (4, 8, True, "fp8"), (4, 12, False, "fp8")])
def test_kv_compress_ex(m, span, per_channel, odt):
    say(f"kv_compress_ex m={m} span={span} per_channel={per_channel} out={odt}")
    g = torch.Generator().manual_seed(1000 * m + span + 7 * per_channel)
    B, T, D = 2, 8 * m + 3 if m < 128 else 1024 + 70, 128
    x = torch.randn(B, T, D, generator=g).to(torch.bfloat16)
    x[0, : 2 * m] *= 1e-3  # small-magnitude entries
    gate = torch.randn((B, T, D) if per_channel else (B, T), generator=g) * 2
    ref = oracle.kv_compress_ex(x, gate, m, span)
    if odt == "fp8":
        codes, scale = cakv.kv_compress_ex(_d(x), _d(gate), m, span, out_dtype=torch.float8_e4m3fn)
        codes, scale = codes.view(torch.uint8).cpu().numpy(), scale.cpu().numpy()
        codes_ref, scale_ref = oracle.q8_quantize(ref)
        deq = oracle.q8_dequantize(codes, scale).astype(np.float64)
        deq_ref = oracle.q8_dequantize(codes_ref, scale_ref).astype(np.float64)
        same = scale == scale_ref
        assert same.mean() > 0.99
        assert np.all(np.isin(scale[~same] / scale_ref[~same], [0.5, 2.0]))
        step = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(deq_ref) / scale_ref[..., None], 2.0 ** -6))) - 3)
        step = np.maximum(step, 2.0 ** -9) * np.maximum(scale, scale_ref)[..., None]
        assert np.all(np.abs(deq - deq_ref) <= step * 1.0001)
        return
    tdt = torch.float32 if odt == "f32" else torch.bfloat16
    out = cakv.kv_compress_ex(_d(x), _d(gate), m, span, out_dtype=tdt).float().cpu().numpy()
    n = _span_tokens(T, m, span)[None, :, None]
    bound = (2 * n + 10) * 2.0 ** -24 * oracle.kv_compress_ex(x.abs(), gate, m, span)
    if odt == "bf16":
        bound = bound + _bf16_ulp(ref)
    err = np.abs(out - ref)
    say(f"  worst error / bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound)


def test_kv_compress_ex_plain_case_is_kv_compress():
    g = torch.Generator().manual_seed(3)
    x = torch.randn(2, 1030, 512, generator=g).to(torch.bfloat16)
    gate = torch.randn(2, 1030, generator=g)
    for m in (4, 128):
        a = cakv.kv_compress(_d(x), _d(gate), m)
        b = cakv.kv_compress_ex(_d(x), _d(gate), m, m)
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ------------------------------------------------------------------ streaming decode

class _Layer:
    """One layer's streaming state on the GPU for B sequences: raw ring,
    gate ring, window ring and compressed cache (prepared entries), plus for
    CSA the indexer key state (raw key ring, gate ring, key cache: fp8 codes
    and scales, or f32 keys)."""

    def __init__(self, B, D, N, m, span, Rr, Rw, per_channel, dt, dI=None, kdt=None):
        self.m, self.span, self.Rr = m, span, Rr
        self.raw = torch.zeros(B, Rr, D, dtype=dt, device=DEV)
        self.graw = torch.zeros((B, Rr, D) if per_channel else (B, Rr), dtype=torch.float32, device=DEV)
        self.win = torch.zeros(B, Rw, D, dtype=dt, device=DEV)
        self.cache = torch.zeros(B, N, D, dtype=dt, device=DEV)
        self.kscale = None
        if dI:
            self.kraw = torch.zeros(B, 8, dI, dtype=kdt, device=DEV)
            self.kgraw = torch.zeros(B, 8, dtype=torch.float32, device=DEV)
            if kdt == torch.float32:
                self.kcache = torch.zeros(B, N, dI, dtype=torch.float32, device=DEV)
            else:
                self.kcache = torch.zeros(B, N, dI, dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn)
                self.kscale = torch.zeros(B, N, dtype=torch.float32, device=DEV)


def _stream_case(name):
    if name == "v4_shapes_after_prefill":
        # a prefill of about 8K tokens by the bulk calls, then 260 streamed
        # tokens per sequence (every sequence crosses two HCA block ends)
        return dict(B=4, H=128, D=512, r=64, n_win=128, HI=64, dI=128, k=128, dt=torch.bfloat16, kdt=torch.bfloat16,
                    prefix=[8000, 8037, 8130, 8003], starts=[0, 0, 0, 0], steps=260, csa_span=4, pc=False, Rr=128)
    # cold start at different positions per sequence; the compressor
    # variants on the CSA KV (span 2m, per-channel gates); fp32 indexer
    return dict(B=3, H=16, D=128, r=32, n_win=16, HI=8, dI=32, k=32, dt=torch.bfloat16, kdt=torch.float32,
                prefix=[0, 0, 0], starts=[0, 5, 61], steps=300, csa_span=8, pc=True, Rr=128)


def _bulk_prefix(lay, b, P, raw, gate, m, span, prep, n_win, kraw=None, kgate=None, hca=False):
    """The state the streaming calls expect after positions 0 .. P-1 of
    sequence b, written by the bulk calls: whole blocks compressed (and
    prepared) into the cache, the last tokens in the rings."""
    if P == 0:
        return
    nb = P // m
    if nb:
        # (per-sequence slices are cloned: every pointer the library takes is 16-byte aligned)
        ent = cakv.kv_compress_ex(raw[b:b + 1, :P].clone(), gate[b:b + 1, :P].clone(), m, span)
        lay.cache[b:b + 1, :nb] = cakv.kv_prepare(ent, m=m, **prep)
    p = torch.arange(max(0, P - lay.Rr), P, device=DEV)
    lay.raw[b, p % lay.Rr] = raw[b, p]
    lay.graw[b, p % lay.Rr] = gate[b, p]
    pw = torch.arange(max(0, P - n_win), P, device=DEV)
    lay.win[b, pw % n_win] = cakv.kv_prepare(raw[b:b + 1, pw].contiguous(), m=1, rope_dims=prep["rope_dims"],
                                             rope_base=prep["rope_base"], entry_pos_offset=int(pw[0]))[0]
    if kraw is not None:
        if nb:
            if lay.kscale is not None:
                kc, ks = cakv.kv_compress(kraw[b:b + 1, :P].clone(), kgate[b:b + 1, :P].clone(), m,
                                          out_dtype=torch.float8_e4m3fn)
                lay.kcache[b:b + 1, :nb] = kc
                lay.kscale[b:b + 1, :nb] = ks
            else:
                lay.kcache[b:b + 1, :nb] = cakv.kv_compress(kraw[b:b + 1, :P].clone(), kgate[b:b + 1, :P].clone(), m,
                                                            torch.float32)
        pk = torch.arange(max(0, P - 8), P, device=DEV)
        lay.kraw[b, pk % 8] = kraw[b, pk]
        lay.kgraw[b, pk % 8] = kgate[b, pk]


@pytest.mark.parametrize("name", ["v4_shapes_after_prefill", "cold_start_overlap_per_channel"])
def test_streaming_decode_steps(name):
    c = _stream_case(name)
    B, H, D, r, n_win, HI, dI, k, dt = c["B"], c["H"], c["D"], c["r"], c["n_win"], c["HI"], c["dI"], c["k"], c["dt"]
    fp8 = c["kdt"] != torch.float32
    m, mh = 4, 128
    prefix, starts = np.array(c["prefix"]), np.array(c["starts"])
    S = c["steps"] + int(starts.max())
    T = int((prefix - starts).max()) + S  # positions that exist in any sequence's raw stream
    say(f"streaming decode {name}: B={B} H={H} D={D} prefix {prefix.tolist()}, {S} steps, CSA span "
        f"{c['csa_span']}, per-channel gates {c['pc']}, indexer {'fp8' if fp8 else 'fp32'}")
    g = torch.Generator().manual_seed(17)
    raw = torch.randn(B, T, D, generator=g).to(dt)
    gate_c = torch.randn((B, T, D) if c["pc"] else (B, T), generator=g)
    gate_h = torch.randn(B, T, generator=g)
    kraw = torch.randn(B, T, dI, generator=g).to(c["kdt"])
    kgate = torch.randn(B, T, generator=g)
    q = torch.randn(B, S, H, D, generator=g).to(dt)  # the step's query
    qh = torch.randn(B, S, H, D, generator=g).to(dt)
    q_idx = torch.randn(B, S, HI, dI, generator=g).to(dt if fp8 else torch.float32)
    w_idx = torch.randn(B, S, HI, generator=g)
    sinks = torch.randn(H, generator=g)
    sinks_h = torch.randn(H, generator=g)
    prep = dict(rope_dims=r, rope_base=10000.0, entry_pos_offset=0, rms_eps=1e-6)
    kw = dict(n_win=n_win, rope_dims=r, rope_base=10000.0)

    N, Nh = T // m, T // mh
    csa = _Layer(B, D, N, m, c["csa_span"], c["Rr"], n_win, c["pc"], dt, dI=dI, kdt=c["kdt"])
    hca = _Layer(B, D, Nh, mh, mh, c["Rr"], n_win, False, dt)
    dev = dict(raw=_d(raw), gate_c=_d(gate_c), gate_h=_d(gate_h), kraw=_d(kraw), kgate=_d(kgate))
    for b in range(B):
        _bulk_prefix(csa, b, int(prefix[b]), dev["raw"], dev["gate_c"], m, c["csa_span"], prep, n_win,
                     kraw=dev["kraw"], kgate=dev["kgate"])
        _bulk_prefix(hca, b, int(prefix[b]), dev["raw"], dev["gate_h"], mh, mh, prep, n_win)
    # the oracle's caches over each full raw stream (visibility masks the future)
    kvc_ref = torch.from_numpy(oracle.kv_compress_ex(raw, gate_c, m, c["csa_span"]).astype(np.float32)).to(dt)
    kvh_ref = torch.from_numpy(oracle.kv_compress(raw, gate_h, mh).astype(np.float32)).to(dt)
    raw0 = torch.zeros(B, dtype=torch.int32)
    qd, qhd, qid, wd = _d(q), _d(qh), _d(q_idx), _d(w_idx)
    sinks_d, sinks_hd = _d(sinks), _d(sinks_h)
    recalls, worst = [], dict(csa=0.0, hca=0.0)
    ar = torch.arange(B)
    for s in range(S):
        t = prefix + s - starts  # sequence b's position at this step (below its prefix: not started)
        live = s >= starts
        t = np.where(live, t, -1)
        tt = np.maximum(t, 0)
        pos = torch.from_numpy(t.astype(np.int32)).to(DEV)
        x_tok = dev["raw"][ar, tt].contiguous()
        cakv.kv_append(x_tok, dev["gate_c"][ar, tt].contiguous(), pos, csa.raw, csa.graw, csa.cache, m=m,
                       span=c["csa_span"], win_ring=csa.win, prep=prep)
        cakv.kv_append(dev["kraw"][ar, tt].contiguous(), dev["kgate"][ar, tt].contiguous(), pos, csa.kraw, csa.kgraw,
                       csa.kcache, m=m, cache_scale=csa.kscale)
        cakv.kv_append(x_tok, dev["gate_h"][ar, tt].contiguous(), pos, hca.raw, hca.graw, hca.cache, m=mh,
                       win_ring=hca.win, prep=prep)
        qpos = pos.view(B, 1)
        idx = cakv.indexer_topk(qid[:, s:s + 1].contiguous(), wd[:, s:s + 1].contiguous(), csa.kcache, csa.kscale,
                                qpos, m, k)
        o_c, _ = cakv.sparse_mqa_fwd(qd[:, s:s + 1].contiguous(), csa.cache, idx, csa.win, None, qpos, sinks_d, m=m,
                                     raw_ring=True, out_dtype=torch.float32, **kw)
        o_h, _ = cakv.dense_compressed_mqa_fwd(qhd[:, s:s + 1].contiguous(), hca.cache, hca.win, None, qpos,
                                               sinks_hd, m=mh, raw_ring=True, out_dtype=torch.float32, **kw)
        rows = np.nonzero(live)[0]
        if rows.size == 0:
            continue
        # the oracle on the full prefix: raw rows linear from position 0
        qp = torch.from_numpy(tt.astype(np.int32)).view(B, 1)
        idx_h = idx.cpu().numpy()
        ref_c, _ = oracle.attention(q[:, s:s + 1], kvc_ref, raw, raw0, qp, sinks, idx=idx_h, m=m, **kw)
        ref_h, _ = oracle.attention(qh[:, s:s + 1], kvh_ref, raw, raw0, qp, sinks_h, m=mh, **kw)
        for nm, o, ref in (("csa", o_c, ref_c), ("hca", o_h, ref_h)):
            oo = o.cpu().numpy().reshape(ref.shape)[rows].astype(np.float64)
            rr = ref[rows]
            err = np.abs(oo - rr).max()
            rel = np.linalg.norm(oo - rr) / np.linalg.norm(rr)
            worst[nm] = max(worst[nm], rel)
            assert np.all(np.isfinite(oo)) and err <= 2e-2 and rel <= 5e-3, (nm, s, err, rel)
        # the selection against the oracle's top-k on the same (GPU-written) keys
        if fp8:
            keys = dict(k_code=csa.kcache.view(torch.uint8).cpu().numpy(), k_scale=csa.kscale.cpu().numpy())
        else:
            keys = dict(k_f32=csa.kcache.cpu().numpy())
        sc, nvis = oracle.indexer_scores(q_idx[:, s:s + 1], w_idx[:, s:s + 1], qp, m, **keys)
        want = oracle.topk(sc, nvis, k)
        for b in rows:
            if not fp8:  # the canonical fp32 mode is bit-exact
                assert np.array_equal(idx_h[b, 0], want[b]), (s, b)
                continue
            gs, ws = set(idx_h[b, 0][idx_h[b, 0] >= 0].tolist()), set(want[b][want[b] >= 0].tolist())
            assert len(gs) == len(ws)
            recalls.append(len(gs & ws) / max(len(ws), 1))
            if gs != ws:
                kth = np.sort(sc[b, :nvis[b]].astype(np.float64))[::-1][min(k, nvis[b]) - 1]
                for j in gs ^ ws:
                    assert abs(sc[b, j] - kth) <= 1e-3 * abs(kth)
    say(f"  worst rel-RMS csa {worst['csa']:.2e} hca {worst['hca']:.2e}"
        + (f"; mean recall {np.mean(recalls):.5f}" if fp8 else "; selection bit-exact"))
    if fp8:
        assert np.mean(recalls) >= 0.995

    # the state equals what the bulk calls write over the whole stream, bitwise
    for b in range(B):
        Tb = int(prefix[b] + S - starts[b])  # positions 0 .. Tb-1 exist now
        xb, gcb, ghb = (dev[f][b:b + 1, :Tb].clone() for f in ("raw", "gate_c", "gate_h"))
        nc, nh = Tb // m, Tb // mh
        bulk_c = cakv.kv_prepare(cakv.kv_compress_ex(xb, gcb, m, c["csa_span"]), m=m, **prep)
        assert torch.equal(csa.cache[b:b + 1, :nc].view(torch.int16), bulk_c.view(torch.int16)), b
        bulk_h = cakv.kv_prepare(cakv.kv_compress(xb, ghb, mh), m=mh, **prep)
        assert torch.equal(hca.cache[b:b + 1, :nh].view(torch.int16), bulk_h.view(torch.int16)), b
        if fp8:
            kc, ks = cakv.kv_compress(dev["kraw"][b:b + 1, :Tb].clone(), dev["kgate"][b:b + 1, :Tb].clone(), m,
                                      out_dtype=torch.float8_e4m3fn)
            assert torch.equal(csa.kcache[b:b + 1, :nc].view(torch.uint8), kc.view(torch.uint8)), b
            assert torch.equal(csa.kscale[b:b + 1, :nc], ks), b
        else:
            kc = cakv.kv_compress(dev["kraw"][b:b + 1, :Tb].clone(), dev["kgate"][b:b + 1, :Tb].clone(), m,
                                  torch.float32)
            assert torch.equal(csa.kcache[b:b + 1, :nc], kc), b
        # the window ring holds the last n_win tokens, prepared at their positions
        p = torch.arange(Tb - n_win, Tb, device=DEV)
        bulk_w = cakv.kv_prepare(dev["raw"][b:b + 1, p].contiguous(), m=1, rope_dims=r, rope_base=10000.0,
                                 entry_pos_offset=int(Tb - n_win))
        for lay in (csa, hca):
            assert torch.equal(lay.win[b, p % n_win].view(torch.int16), bulk_w[0].view(torch.int16)), b
        assert torch.equal(csa.raw[b, p % c["Rr"]].view(torch.int16), dev["raw"][b, p].view(torch.int16))
        # entries of blocks not yet complete were never written
        assert not csa.cache[b, nc:].any() and not hca.cache[b, nh:].any()


# ------------------------------------------------------------------ batched appends

# (activations, cache, per-channel gates, prepared entries with a window ring)
_APPEND_KINDS = [
    (torch.float32, torch.float32, False, True), (torch.float32, torch.float32, True, False),
    (torch.float32, torch.float8_e4m3fn, False, False), (torch.float32, torch.float8_e4m3fn, True, False),
    (torch.bfloat16, torch.bfloat16, False, True), (torch.bfloat16, torch.bfloat16, True, True),
    (torch.bfloat16, torch.float8_e4m3fn, False, False), (torch.bfloat16, torch.float8_e4m3fn, True, False),
]


@pytest.mark.parametrize("group", [(0, 1, 2, 3), (4, 5, 6, 7), (5, 6, 4)])
def test_kv_append_batch_matches_separate_calls(group):
    """Every kind of append (f32 or bf16 tokens; a cache of their type or fp8
    codes; one gate logit per token or per channel; prepared entries with a
    window ring, or not) in batches of up to four, over 70 steps with
    sequences that start late (position -1 before) and blocks of 4, 8 and 16
    tokens with spans of one or two blocks: the batched launch leaves every
    ring, cache and scale bitwise as the same appends made one by one."""
    say(f"kv_append_batch, kinds {group}")
    B, D, steps, Rr, Rw = 3, 64, 70, 32, 8
    starts = np.array([0, 3, 10])
    prep = dict(rope_dims=16, rope_base=10000.0, entry_pos_offset=0, rms_eps=1e-6)
    g = torch.Generator().manual_seed(sum(group) + 101)
    cfg, toks = [], []
    for n_, kind in enumerate(group):
        act, cdt, pc, pw = _APPEND_KINDS[kind]
        m = (4, 8, 16, 4)[n_]
        span = m * (1 + n_ % 2)
        N = steps // m
        cfg.append((act, cdt, pc, pw, m, span, N))
        toks.append((torch.randn(steps, B, D, generator=g).to(act),
                     torch.randn((steps, B, D) if pc else (steps, B), generator=g)))

    def state():
        out = []
        for act, cdt, pc, pw, m, span, N in cfg:
            st = dict(raw=torch.zeros(B, Rr, D, dtype=act, device=DEV),
                      graw=torch.zeros((B, Rr, D) if pc else (B, Rr), dtype=torch.float32, device=DEV),
                      win=torch.zeros(B, Rw, D, dtype=act, device=DEV) if pw else None,
                      scale=torch.zeros(B, N, dtype=torch.float32, device=DEV) if cdt == torch.float8_e4m3fn else None)
            st["cache"] = (torch.zeros(B, N, D, dtype=torch.uint8, device=DEV).view(torch.float8_e4m3fn)
                           if cdt == torch.float8_e4m3fn else torch.zeros(B, N, D, dtype=cdt, device=DEV))
            out.append(st)
        return out

    one, bat = state(), state()
    for s in range(steps):
        t = np.where(s >= starts, s - starts, -1).astype(np.int32)
        pos = torch.from_numpy(t).to(DEV)
        calls = []
        for (act, cdt, pc, pw, m, span, N), (x, gt), a, b in zip(cfg, toks, one, bat):
            xs, gs = _d(x[s]), _d(gt[s])
            kw = dict(m=m, span=span, cache_scale=a["scale"], win_ring=a["win"], prep=prep if pw else None)
            cakv.kv_append(xs, gs, pos, a["raw"], a["graw"], a["cache"], **kw)
            calls.append(dict(x_tok=xs, gate_tok=gs, raw_ring=b["raw"], gate_ring=b["graw"], cache=b["cache"], m=m,
                              span=span, cache_scale=b["scale"], win_ring=b["win"], prep=prep if pw else None))
        cakv.kv_append_batch(calls, pos)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(one, bat)):
        for key in ("raw", "graw", "win", "cache", "scale"):
            if a[key] is None:
                continue
            x, y = a[key], b[key]
            if x.dtype == torch.float8_e4m3fn:
                x, y = x.view(torch.uint8), y.view(torch.uint8)
            assert torch.equal(x, y), (group[i], key)
        assert torch.count_nonzero(a["cache"].view(torch.uint8) if a["cache"].dtype == torch.float8_e4m3fn
                                   else a["cache"]) > 0  # entries were written
