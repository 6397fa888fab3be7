"""q4_pack on the GPU: codes and scales byte-identical to the oracle."""

import numpy as np
import pytest

from gpu_util import dev, host, torch_cuda
from oracle import q4
from bit_quantized_weight_amd import pack, synthetic
from test_oracle_q4 import _special_rows

pytestmark = pytest.mark.gpu


def _check(w):
    torch = torch_cuda()
    codes, scales = pack(dev(w, torch))
    torch.cuda.synchronize()
    q, d = q4.quantize(w)
    assert np.array_equal(host(codes), q4.pack(q)), "codes differ"
    assert np.array_equal(host(scales).view(np.uint16), d.view(np.uint16)), "scales differ"


@pytest.mark.parametrize("n,k,seed", [(512, 256, 0), (17, 96, 3), (1, 32, 4), (333, 544, 5), (7, 17408, 6)])
def test_pack_bit_exact(n, k, seed):
    _check(synthetic.weights(n, k, seed))


def test_pack_special_blocks():
    """Exact ties, zero blocks, fp16-subnormal and zero-rounding scales."""
    _check(_special_rows())


def test_pack_wide_range():
    rng = np.random.default_rng(9)
    mags = 10.0 ** rng.uniform(-8, 4, size=(64, 1))
    _check((rng.standard_normal((64, 256)) * mags).astype(np.float32))


def test_pack_all_ones_closed_form():
    torch = torch_cuda()
    codes, scales = pack(torch.ones((4, 5120), dtype=torch.float32, device="cuda"))
    assert np.all(host(scales).astype(np.float64) == 0.142822265625)
    assert np.all(host(codes) == 0x77)


def test_pack_decode_shape():
    """The decode gate/up matrix, 17408 x 5120, about 8 exact rounding ties."""
    _check(synthetic.weights(17408, 5120, synthetic.WEIGHT_SEED))


def test_pack_empty():
    torch = torch_cuda()
    codes, scales = pack(torch.zeros((0, 64), dtype=torch.float32, device="cuda"))
    assert codes.shape == (0, 32) and scales.shape == (0, 2)


def test_pack_in_pieces():
    """More than 2^26 blocks (N = 65600, K = 32768: 67,174,400 blocks, 8.6 GB of
    fp32 input) are packed in two launches that split at block 2^26, the first
    block of row 65536; rows on both sides of the split and the last row match
    the oracle byte for byte."""
    torch = torch_cuda()
    n, k = 65600, 32768
    w = synthetic.weights_device(n, k, 31)
    codes, scales = pack(w)
    torch.cuda.synchronize()
    rows = [0, 65535, 65536, 65537, n - 1]
    sel = torch.as_tensor(rows, device="cuda")
    wr = w.index_select(0, sel).cpu().numpy()
    c = codes.index_select(0, sel).cpu().numpy()
    s = scales.index_select(0, sel).cpu().numpy()
    del w, codes, scales
    q, d = q4.quantize(wr)
    assert np.array_equal(c, q4.pack(q)), "codes differ"
    assert np.array_equal(s.view(np.uint16), d.view(np.uint16)), "scales differ"
