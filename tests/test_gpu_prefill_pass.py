"""Full 64-layer prefill weight pass on the A8 route at M = 2048 tokens:
sampled tokens x sampled output rows of the first and last layers against the
A8 oracle, and a repeated pass bit-identical to the first."""

import numpy as np
import pytest

from gpu_util import assert_close, host, torch_cuda
from oracle import a8, q4
from bit_quantized_weight_amd import synthetic
from bit_quantized_weight_amd.prefill import PrefillPass

pytestmark = pytest.mark.gpu

M = 2048
CHECK_LAYERS = (0, synthetic.N_LAYERS - 1)
INPUT_OF = {"qkv": 0, "out": 1, "gate": 0, "up": 0, "down": 2}


def _rows(n, seed, count=24):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, count)]))


TOKENS = _rows(M, 5, 14)


@pytest.fixture(scope="module")
def prefill_pass():
    torch = torch_cuda()
    keep = {(layer, pi): _rows(n, 100 * layer + pi)
            for layer in CHECK_LAYERS
            for pi, (_, _, n) in enumerate(synthetic.LAYER_PROJECTIONS)}
    p = PrefillPass(M, keep_rows=keep)
    yield p
    del p
    torch.cuda.empty_cache()


def _check_layer(p, layer):
    xs = [host(x) for x in p.xs]
    for pi, (name, k, n) in enumerate(synthetic.LAYER_PROJECTIONS):
        rows = _rows(n, 100 * layer + pi)
        q, d = q4.quantize(p.kept[(layer, pi)])
        ref = a8.prefill(xs[INPUT_OF[name]][TOKENS], q, d)      # [tokens, rows]
        got = host(p.ys[pi])[TOKENS][:, rows]
        assert_close(got, ref, what=f"prefill layer {layer} {name}")


def test_prefill_first_layer(prefill_pass):
    torch = torch_cuda()
    prefill_pass.run(layers=[0])
    torch.cuda.synchronize()
    _check_layer(prefill_pass, 0)


def test_prefill_whole_pass_and_repeat(prefill_pass):
    """The whole pass leaves the last layer's outputs; a second pass gives the
    same bits (fixed order of every sum)."""
    torch = torch_cuda()
    prefill_pass.run()
    torch.cuda.synchronize()
    _check_layer(prefill_pass, CHECK_LAYERS[-1])
    first = [host(y).copy() for y in prefill_pass.ys]
    for y in prefill_pass.ys:
        y.fill_(7.0)
    prefill_pass.run()
    torch.cuda.synchronize()
    for pi, (a, y) in enumerate(zip(first, prefill_pass.ys)):
        assert np.array_equal(a.view(np.uint16), host(y).view(np.uint16)), pi
