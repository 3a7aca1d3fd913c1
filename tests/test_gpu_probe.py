"""The streaming-read probe the benchmark uses for its practical peak reads
every 16-byte unit exactly once: the XOR of its per-workgroup words equals
the XOR of all the buffer's 32-bit words."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words,blocks", [(4 * 1000003, 64), (4 * 4096, 4096), (4, 3)])
def test_stream_read_probe_reads_every_unit_once(n_words, blocks):
    from sparse_long_context_compressor_amd import slc
    g = torch.Generator().manual_seed(n_words)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (n_words,), generator=g, dtype=torch.int64).to(torch.int32)
    buf = host.cuda()
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    slc.stream_read_probe(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want
