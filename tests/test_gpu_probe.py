"""The streaming-read probe the benchmark uses for its practical peak
(bench_probe.hip, measurement only) reads every 16-byte unit exactly once:
the XOR of its per-workgroup words equals the XOR of all the buffer's
32-bit words."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_words,blocks", [(4 * 1000003, 64), (4 * 4096, 4096), (4, 3),
                                            (4 * 8 * 256 * 5 + 12, 5)])
def test_stream_read_probe_reads_every_unit_once(n_words, blocks):
    import bench
    g = torch.Generator().manual_seed(n_words)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (n_words,), generator=g, dtype=torch.int64).to(torch.int32)
    buf = host.cuda()
    sink = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    bench.stream_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want
