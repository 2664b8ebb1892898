"""The allocation-free indexer entry point, cakv_indexer_topk_noalloc, called
through the C ABI: on two calls in a row, the second with a smaller input
(and the other indexer mode), it returns bitwise what cakv_indexer_topk
returns with a workspace, and what the oracle requires (fp8 mode: recall and
gap bar; fp32 mode: bit-exact).  Sizes beyond its static scratch are refused
on the host."""
import numpy as np
import pytest
import torch

import compressed_attention_kv_amd as cakv
import oracle

DEV = "cuda:0"


def _d(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _case(seed, B, Q, N, HI, dI, fp8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Q, HI, dI)).astype(np.float32)
    w = rng.standard_normal((B, Q, HI)).astype(np.float32)
    keys = rng.standard_normal((B, N, dI)).astype(np.float32)
    qpos = np.full((B, Q), 4 * N, dtype=np.int32)
    qpos[0, 0] = 4 * N // 3  # fewer visible entries in one row
    if fp8:
        qb = torch.from_numpy(q).to(torch.bfloat16)
        codes, scale = oracle.q8_quantize(keys)
        return dict(q=qb, w=w, keys=codes, scale=scale, qpos=qpos)
    return dict(q=torch.from_numpy(q), w=w, keys=keys, scale=None, qpos=qpos)


@pytest.mark.gpu
def test_noalloc_matches_the_workspace_entry_point():
    calls = [dict(seed=1, B=8, Q=1, N=65536, HI=64, dI=128, k=1024, fp8=True),
             dict(seed=2, B=2, Q=3, N=5000, HI=8, dI=32, k=256, fp8=False)]  # smaller, fp32 mode
    for c in calls:
        print(f"noalloc indexer {c}", flush=True)
        inp = _case(c["seed"], c["B"], c["Q"], c["N"], c["HI"], c["dI"], c["fp8"])
        args = (inp["q"].to(DEV), _d(inp["w"]), _d(inp["keys"]), None if inp["scale"] is None else _d(inp["scale"]),
                _d(inp["qpos"]), 4, c["k"])
        ref = cakv.indexer_topk(*args)
        out = torch.full((c["B"], c["Q"], c["k"]), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
        got = cakv.indexer_topk_noalloc(*args, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got, ref)
        g = got.cpu().numpy().reshape(c["B"] * c["Q"], c["k"])
        if c["fp8"]:
            scores, nvis = oracle.indexer_scores(inp["q"], inp["w"], inp["qpos"], 4, k_code=inp["keys"],
                                                 k_scale=inp["scale"])
            want = oracle.topk(scores, nvis, c["k"])
            recall = np.mean([len(set(a[a >= 0]) & set(b[b >= 0])) / max((b >= 0).sum(), 1)
                              for a, b in zip(g, want)])
            print(f"  recall {recall:.5f}", flush=True)
            assert recall >= 0.995
        else:
            want = oracle.indexer_topk(inp["q"], inp["w"], inp["qpos"], 4, c["k"], k_f32=inp["keys"])
            assert np.array_equal(g, want)


def test_noalloc_refuses_sizes_beyond_its_scratch():
    lib = cakv.load_library()
    FAKE = 0x10000
    f = lib.cakv_indexer_topk_noalloc
    # 1000 queries over 262,144 entries need about 1 GB of workspace
    assert lib.cakv_indexer_topk_workspace(1000, 1, 262144, 1024) > (64 << 20)
    rc = f(FAKE, cakv.BF16, FAKE, FAKE, cakv.FP8_E4M3, FAKE, FAKE, 1000, 1, 262144, 64, 128, 4, 1024, FAKE, None)
    assert rc == -3
    assert "scratch" in lib.cakv_last_error().decode()
    # argument errors are the workspace call's; an empty batch does nothing
    assert f(FAKE, cakv.BF16, FAKE, FAKE, cakv.FP8_E4M3, FAKE, FAKE, 1, 1, 64, 48, 128, 4, 16, FAKE, None) == -2
    assert f(None, cakv.BF16, None, None, cakv.FP8_E4M3, None, None, 0, 1, 64, 64, 128, 4, 16, None, None) == 0
