"""Parity at the documented maximum sizes, against the oracle and to the bars
of the tests they extend: the compressor at D = 4,096 (the short-span run
kernel's several workgroup columns, the general kernel's 256-thread entries)
and at the longest block, m = 4,096; the compressor variants at D = 4,096
with per-channel gates and at the longest span, 8,192; the sparse attention
over K = 65,536 selected entries with the longest window, n_win = 4,096."""
import sys

import numpy as np
import pytest
import torch

import compressed_attention_kv_amd as cakv
import oracle

import test_parity_gpu as P
import test_stream_gpu as S

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dtype,D,m,T", [("bf16", 4096, 4, 8 * 4 + 3), ("f32", 4096, 4, 70),
                                         ("bf16", 4096, 128, 2 * 128 + 5), ("f32", 64, 4096, 2 * 4096 + 9)])
def test_kv_compress_max_sizes(dtype, D, m, T):
    P.test_kv_compress(dtype, D, m, T)


@pytest.mark.parametrize("m,span,per_channel,odt", [(4, 8192, False, "bf16"), (128, 8192, True, "f32")])
def test_kv_compress_ex_longest_span(m, span, per_channel, odt):
    S.test_kv_compress_ex(m, span, per_channel, odt)


@pytest.mark.parametrize("span,odt", [(8, "bf16"), (4, "f32")])
def test_kv_compress_ex_widest_rows(span, odt):
    say(f"kv_compress_ex D=4096 span={span} per-channel out={odt}")
    g = torch.Generator().manual_seed(4096 + span)
    B, T, D, m = 2, 4 * 21 + 3, 4096, 4
    x = torch.randn(B, T, D, generator=g).to(torch.bfloat16)
    gate = torch.randn(B, T, D, generator=g) * 2
    ref = oracle.kv_compress_ex(x, gate, m, span)
    tdt = torch.float32 if odt == "f32" else torch.bfloat16
    out = cakv.kv_compress_ex(S._d(x), S._d(gate), m, span, out_dtype=tdt).float().cpu().numpy()
    n = S._span_tokens(T, m, span)[None, :, None]
    bound = (2 * n + 10) * 2.0 ** -24 * oracle.kv_compress_ex(x.abs(), gate, m, span)
    if odt == "bf16":
        bound = bound + S._bf16_ulp(ref)
    err = np.abs(out - ref)
    say(f"  worst error / bound {np.max(err / bound):.3f}")
    assert np.all(err <= bound)


def test_sparse_attention_largest_selection_and_window():
    say("sparse attention, K = 65,536 and n_win = 4,096")
    g = torch.Generator().manual_seed(21)
    B, Q, H, D, K, n_win = 1, 2, 8, 512, 65536, 4096
    N = K + 100
    t = 4 * N + 7
    q = torch.randn(B, Q, H, D, generator=g).to(torch.bfloat16)
    kv = torch.randn(B, N, D, generator=g).to(torch.bfloat16)
    raw = torch.randn(B, n_win, D, generator=g).to(torch.bfloat16)
    sinks = torch.randn(H, generator=g)
    qpos = torch.tensor([[t, t - 1000]], dtype=torch.int32)  # the second query reaches past the raw rows' start
    raw0 = torch.tensor([t - n_win + 1], dtype=torch.int32)
    idx = torch.stack([torch.randperm(N, generator=g)[:K] for _ in range(Q)]).view(B, Q, K).to(torch.int32)
    idx[:, :, ::97] = -1
    kw = dict(m=4, n_win=n_win, rope_dims=64)
    ref, lse_ref = oracle.attention(q, kv, raw, raw0, qpos, sinks, idx=idx.numpy(), **kw)
    kvp, rawp = P._prep(kv, 4, kw), P._prep_raw(raw, raw0, kw)
    out, lse = cakv.sparse_mqa_fwd(P._d(q), kvp, P._d(idx), rawp, P._d(raw0), P._d(qpos), P._d(sinks),
                                   out_dtype=torch.float32, **kw)
    P._attn_check(out.cpu().numpy().reshape(ref.shape), ref, "K = 65,536")
    lg = lse.cpu().numpy().reshape(lse_ref.shape)
    assert np.abs(lg - lse_ref).max() < 1e-2  # bf16 logits
