"""The roofline probes (measurement support): the streaming read touches
every word of its buffer once, and the matrix-core loop runs."""
import pytest
import torch

import quantized_moe_expert_02_amd as moe

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words,blocks", [(1 << 18, 64), ((1 << 18) + 12, 37), (4, 1)])
def test_stream_read_reads_every_word(n_words, blocks):
    g = torch.Generator().manual_seed(n_words + blocks)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (n_words,), generator=g, dtype=torch.int64).to(torch.int32)
    buf = host.cuda()
    sink = torch.zeros(blocks * 256, dtype=torch.int32, device="cuda")
    moe.probe_stream_read(buf, blocks, sink)
    torch.cuda.synchronize()
    want = 0
    for v in host.view(torch.int32).tolist():
        want ^= v & 0xFFFFFFFF
    got = 0
    for v in sink.cpu().tolist():
        got ^= v & 0xFFFFFFFF
    assert got == want


def test_mfma_probe_runs():
    sink = torch.zeros(8 * 512, dtype=torch.int32, device="cuda")
    flops = moe.probe_mfma(sink, 8, 10)
    torch.cuda.synchronize()
    vals = sink.view(torch.float32)
    assert flops == 8 * 8 * 10 * 16 * 16384
    assert torch.isfinite(vals).all() and (vals > 0).all()
