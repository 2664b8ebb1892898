"""The debug build (kernels compiled with -DCAKV_DEBUG: device-side checks
of their own index invariants, e.g. the top-k's k distinct in-range winners,
the XCD mapping's range, the streaming append's span inside its ring) runs a
selection of the parity tests, each against the oracle as in its own module:
the compressor (both kernels), the indexer's select paths (including tied
blocks at the k-th place), sparse and dense attention with splits and edge
cases, the streaming append (one call and batched) and the indexer backward.  The binding's cached
library is swapped for the debug one for the length of each test.  Skipped
when the debug build is absent (python -m compressed_attention_kv_amd.build
--debug, which __graft_entry__.build() also runs)."""
import os

import pytest

import compressed_attention_kv_amd as cakv
from compressed_attention_kv_amd import build as hipbuild

import test_backward_gpu as BW
import test_parity_gpu as P
import test_stream_gpu as S

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def debug_library(monkeypatch):
    if not os.path.exists(hipbuild.DEBUG_LIB):
        pytest.skip("the debug build is absent")
    cakv.load_library()  # the regular build stays cached for the other modules
    monkeypatch.setattr(cakv, "_lib", None)
    lib = cakv.load_library(hipbuild.DEBUG_LIB)
    assert lib._name == hipbuild.DEBUG_LIB
    yield lib


@pytest.mark.parametrize("dtype,D,m,T", [("f32", 128, 4, 2048), ("bf16", 512, 4, 8192 + 7), ("bf16", 512, 128, 8192)])
def test_debug_kv_compress(dtype, D, m, T):
    P.test_kv_compress(dtype, D, m, T)


def test_debug_kv_compress_fp8():
    P.test_kv_compress_fp8(8192 + 3, 4)


def test_debug_indexer_select_paths():
    P.test_indexer_fp32_bit_exact_tiny_layer()
    P.test_indexer_fp32_bit_exact_sizes(3000, 64, 8)
    for tied in (3000, 5000, 10000):
        P.test_indexer_fp32_tied_block_at_threshold(tied)
        P.test_indexer_fp8_fused_refine_matches(tied)


def test_debug_attention():
    P.test_sparse_attention_tiny_layer_f32()
    P.test_dense_attention_tiny_hca_f32()
    P.test_attention_edge_cases()
    P.test_attention_split_combine_odd_heads()


def test_debug_compressor_variants_and_streaming():
    S.test_kv_compress_ex(4, 8, True, "bf16")
    S.test_streaming_decode_steps("cold_start_overlap_per_channel")
    S.test_kv_append_batch_matches_separate_calls((4, 5, 6, 7))


def test_debug_indexer_fp8_whole_line_loads():
    P.test_indexer_fp8_whole_line_loads_match(32768 + 77, 1024, 64, 128)
    P.test_indexer_fp8_whole_line_loads_match(9000, 512, 32, 128)
    P.test_indexer_fp8_whole_line_loads_match(7000 + 5, 256, 64, 64)


def test_debug_indexer_backward():
    BW.test_indexer_backward("fp8", BW.INDEXER_BWD_SHAPES[1])
