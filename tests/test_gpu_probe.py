"""The streaming-read probe (a measurement helper) reads every byte once:
the XOR of its per-thread checksums equals the XOR of the buffer's words."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
cq = pytest.importorskip("hadamard_rotated_codebook_amd")


@pytest.mark.parametrize("nbytes,groups", [(1 << 20, 64), ((1 << 20) + 4096 + 16, 8), (48, 1), (285212672, 2048)])
def test_read_probe_reads_every_byte_once(nbytes, groups):
    g = torch.Generator(device="cuda:0")
    g.manual_seed(nbytes)
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g, device="cuda:0")
    sink = torch.empty(groups * 256, dtype=torch.int32, device="cuda:0")
    cq.cq_read_probe(buf, sink)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32))
    assert got == want
