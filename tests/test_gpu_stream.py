"""GPU: the read-only streaming kernel behind the bench's HBM read ceiling reads every 16-byte word
of its buffer exactly once: the XOR of the per-workgroup words it writes equals the XOR of all
32-bit words of the buffer (bit-exact, numpy on the host), for sizes that leave ragged tails of
the unrolled grid-stride loop."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU boxes only to be deselected by -m "not gpu"
    pytest.skip("no GPU", allow_module_level=True)

import mla_latent_kv_25_amd as mla  # noqa: E402


@pytest.mark.parametrize("n16", [1, 7, 256, 2048 * 8 + 5, 1 << 20, (1 << 22) + 333])
def test_stream_read_xor(n16):
    g = torch.Generator(device="cpu").manual_seed(77 + n16)
    host = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), generator=g, dtype=torch.int64).to(torch.int32)
    src = host.cuda()
    sink = torch.zeros(mla.STREAM_SINK_WORDS, dtype=torch.int32, device="cuda")
    mla.stream_read(src, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert got == want
