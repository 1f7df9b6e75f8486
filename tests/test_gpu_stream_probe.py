"""GPU check of the streaming-read probe (the bandwidth measurement helper):
every 32-bit word of the source is folded into exactly one wave's checksum,
so the XOR of all checksums equals the XOR of the whole buffer, for sizes
that split unevenly over the CUs and leave ragged last steps."""
import numpy as np
import pytest

from _helpers import need_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, (7 << 20) + 48, 64 << 20])
def test_stream_probe_reads_every_word_once(nbytes):
    need_gpu()
    import torch
    import quantized_moe_weight_amd as pq
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda", generator=g)
    sink = torch.zeros(16384, dtype=torch.int32, device="cuda")
    pq.stream_probe(src, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want
