"""GPU check of the read-stream reference kernel (lbp_read_stream): every
workgroup's digest is the XOR of the 32-bit words of its chunk, so the kernel
read every byte once (bit-exact, against NumPy)."""

import numpy as np
import pytest
import torch

import load_balanced_paged_amd as lbp
from gpu_support import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16,blocks", [(1 << 22, 1), (1 << 22, 7), (1 << 22, 1024), (1000, 300)])
def test_read_stream_digests(gpu_lib, n16, blocks):
    say(f"[stream] n16={n16} blocks={blocks}")
    g = torch.Generator(device="cuda").manual_seed(n16 + blocks)
    buf = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), generator=g, dtype=torch.int32,
                        device="cuda")
    sink = torch.full((blocks,), -1, dtype=torch.int32, device="cuda")
    lbp.lbp_read_stream(buf, sink, blocks)
    torch.cuda.synchronize()
    words = buf.cpu().numpy().reshape(n16, 4)
    per = -(-n16 // blocks)
    want = np.zeros(blocks, dtype=np.int32)
    for b in range(blocks):
        chunk = words[b * per:min(n16, (b + 1) * per)]
        if len(chunk):
            want[b] = np.bitwise_xor.reduce(chunk.ravel())
    assert np.array_equal(sink.cpu().numpy(), want)
