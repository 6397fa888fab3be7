"""The binding refuses packed weights or caches whose shapes do not match the
activations (the library would read exactly the implied sizes), before any
launch."""

import pytest

from gpu_util import torch_cuda
from bit_quantized_weight_amd import a8w4_gemm, attn_decode, batched_plan, gemv, gemv_noalloc, pack, synthetic

pytestmark = pytest.mark.gpu


def _packed(torch, n, k, seed):
    return pack(synthetic.weights_device(n, k, seed))


def test_weight_shapes_are_checked():
    torch = torch_cuda()
    codes, scales = _packed(torch, 64, 256, 1)
    x = synthetic.activations_device(2, 512, 2)                 # K = 512, weights packed for 256
    with pytest.raises(ValueError):
        gemv(x, codes, scales)
    with pytest.raises(ValueError):
        a8w4_gemm(x, codes, scales)
    y = torch.empty((2, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        gemv_noalloc(x, codes, scales, y)
    x2 = synthetic.activations_device(2, 256, 3)
    with pytest.raises(ValueError):                             # scales of another matrix
        gemv(x2, codes, scales[:32])
    with pytest.raises(ValueError):                             # y of the wrong width
        batched_plan([(x2, codes, scales, torch.empty((2, 32), dtype=torch.float16, device="cuda"))])
    torch.cuda.synchronize()
    assert gemv(x2, codes, scales).shape == (2, 64)


def test_cache_shapes_are_checked():
    torch = torch_cuda()
    kc, ks = _packed(torch, 100, 4 * 256, 4)
    vc, vs = _packed(torch, 99, 4 * 256, 5)                     # one row short
    q = synthetic.activations_device(2 * 20, 256, 6).reshape(2, 20, 256)
    with pytest.raises(ValueError):
        attn_decode(q, kc, ks, vc, vs, 4)
    with pytest.raises(ValueError):                             # caches for 2 K/V heads, 4 claimed
        kc2, ks2 = _packed(torch, 100, 2 * 256, 7)
        attn_decode(q, kc2, ks2, kc2, ks2, 4)
    torch.cuda.synchronize()
    assert attn_decode(q, kc, ks, kc, ks, 4).shape == (2, 20, 256)
