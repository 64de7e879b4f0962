"""GPU test of dh_stream_read, the streaming-read diagnostic the benchmark reports as the
device's practical read bandwidth: its sink must sum (mod 2^32) to the sum of the buffer's
32-bit words, so every byte is read exactly once, at sizes from one 4 KiB segment to more
segments than the grid has waves; sizes that are not whole segments are refused."""
import numpy as np
import pytest
import torch

from few_row_vocab_amd import dh
from gpu_util import host, need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [4096, 3 * 4096, 1 << 20, 64 * (1 << 20) + 4096])
def test_stream_read_reads_every_byte_once(nbytes):
    need_gpu()
    say(f"stream read {nbytes} bytes")
    g = torch.Generator(device="cuda").manual_seed(nbytes % 1000)
    buf = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    sink = dh.stream_read(buf)
    torch.cuda.synchronize()
    want = int(host(buf).view(np.uint32).astype(np.uint64).sum()) % (1 << 32)
    got = int(host(sink).view(np.uint32).astype(np.uint64).sum()) % (1 << 32)
    assert got == want


def test_stream_read_refusals():
    need_gpu()
    buf = torch.zeros((4096 + 100,), dtype=torch.uint8, device="cuda")
    with pytest.raises(dh.DHError):
        dh.stream_read(buf)                                   # not whole 4 KiB segments
    with pytest.raises(dh.DHError):
        dh.stream_read(buf[1:4097])                           # misaligned
