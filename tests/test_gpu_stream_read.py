"""q4w_stream_read, the plain-read helper whose rate the bench reports as the
achievable ceiling: its checksum (XOR of every 32-bit word) must match the
host's for any launch shape, so every byte is read exactly once."""

import numpy as np
import pytest

from gpu_util import host, torch_cuda
from bit_quantized_weight_amd import stream_read

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,grid,block", [(3 * 1024 * 1024 + 48, 256, 512), (1 << 20, 2048, 256),
                                               (16, 1, 64), (4096 + 16, 7, 1024), (0, 3, 64)])
def test_checksum(nbytes, grid, block):
    torch = torch_cuda()
    rng = np.random.default_rng(nbytes + grid)
    data = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(data.view(np.int32)).to("cuda") if nbytes else torch.empty(0, dtype=torch.int32, device="cuda")
    out = stream_read(buf, grid=grid, block=block)
    torch.cuda.synchronize()
    assert out.shape == (grid * (block // 64),)
    got = np.bitwise_xor.reduce(host(out).view(np.uint32))
    want = np.bitwise_xor.reduce(data) if nbytes else np.uint32(0)
    assert int(got) == int(want)
