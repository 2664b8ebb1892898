"""The attainable-peak probes (include/cakv_probes.h) that price the
benchmark's roofline fractions: the streaming read loads every byte of its
buffer exactly once (its per-workgroup XOR checksums combine to the XOR of
the buffer's 32-bit words, computed here by numpy), and the MFMA loop
performs the documented products (with operands of 0.5 every accumulator
of column 0 gains 16 * 0.25 = 4 per round, so each wave's sum of its four
chains' 16 registers is 256 * iters, exactly in fp32)."""
import sys

import numpy as np
import pytest
import torch

import compressed_attention_kv_amd as cakv

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("nbytes,blocks", [((1 << 20) + 48, 7), ((1 << 20) + 48, 0), (16, 3), (4096 * 16, 2048)])
def test_probe_read_checksum(nbytes, blocks):
    say(f"probe_read {nbytes} bytes, {blocks or 2048} workgroups")
    g = np.random.default_rng(nbytes + blocks)
    host = g.integers(0, 256, size=nbytes, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    nb = blocks or 2048
    sink = torch.full((nb,), -1, dtype=torch.int32, device="cuda")
    cakv.probe_read(buf, sink, blocks)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.view(np.uint32))
    assert got == want


def test_probe_read_empty_buffer_zeroes_the_sink():
    say("probe_read, 0 bytes")
    buf = torch.zeros(16, dtype=torch.uint8, device="cuda")
    sink = torch.full((5,), -1, dtype=torch.int32, device="cuda")
    rc = cakv.load_probes().cakv_probe_read(buf.data_ptr(), 0, sink.data_ptr(), 5,
                                            torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    assert torch.all(sink.cpu() == 0)


@pytest.mark.parametrize("iters,blocks", [(100, 3), (0, 1), (4096, 2)])
def test_probe_mfma_closed_form(iters, blocks):
    say(f"probe_mfma_bf16 iters={iters} blocks={blocks}")
    sink = torch.full((4 * blocks,), -1.0, dtype=torch.float32, device="cuda")
    flops = cakv.probe_mfma_bf16(iters, blocks, sink)
    assert flops == blocks * 4 * iters * 4 * 32768
    assert torch.all(sink.cpu() == 256.0 * iters)
