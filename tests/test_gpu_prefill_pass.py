"""Full 64-layer prefill weight pass on the A8 route at M = 512, 1024 and
2048 tokens (the pages' pp512 and pp2048 prompts and the chunk of 1024 used
for long prompts, page 5, "Qwen3.8-27B on RTX 4090: 5,000 tok/s Prefill
Reproduced"): sampled tokens x sampled output rows of the first and last
layers against the A8 oracle (gate and up run as one GEMM), and a repeated
pass bit-identical to the first.  One set of packed weights serves all three
prompt lengths; at M = 512 the qkv, out and down GEMMs take the 64-row tile
form and gate|up the chunk-balanced form, at M = 2048 out and down take the
chunk-balanced form."""

import numpy as np
import pytest

from gpu_util import assert_close, host, torch_cuda
from oracle import a8, q4
from bit_quantized_weight_amd import synthetic
from bit_quantized_weight_amd.prefill import PrefillPass

pytestmark = pytest.mark.gpu

MS = (512, 1024, 2048)
CHECK_LAYERS = (0, synthetic.N_LAYERS - 1)
INPUT_OF = {"qkv": 0, "out": 1, "gate": 0, "up": 0, "down": 2}


def _rows(n, seed, count=24):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, count)]))


def _tokens(m):
    return _rows(m, 5, 14)


@pytest.fixture(scope="module")
def weights_pass():
    """The pass that packs the 64 layers' weights (and keeps the sampled fp32
    rows of the checked layers); the other prompt lengths reuse them."""
    torch = torch_cuda()
    keep = {(layer, pi): _rows(n, 100 * layer + pi)
            for layer in CHECK_LAYERS
            for pi, (_, _, n) in enumerate(synthetic.LAYER_PROJECTIONS)}
    p = PrefillPass(MS[0], keep_rows=keep)
    yield p
    del p
    torch.cuda.empty_cache()


@pytest.fixture(scope="module", params=MS, ids=[f"M{m}" for m in MS])
def prefill_pass(request, weights_pass):
    torch = torch_cuda()
    m = request.param
    if m == weights_pass.m:
        yield weights_pass
        return
    p = PrefillPass(m, weights=weights_pass.layers)
    p.kept = weights_pass.kept
    yield p
    del p
    torch.cuda.empty_cache()


def _check_layer(p, layer):
    xs = [host(x) for x in p.xs]
    tokens = _tokens(p.m)
    for pi, (name, k, n) in enumerate(synthetic.LAYER_PROJECTIONS):
        rows = _rows(n, 100 * layer + pi)
        q, d = q4.quantize(p.kept[(layer, pi)])
        ref = a8.prefill(xs[INPUT_OF[name]][tokens], q, d)      # [tokens, rows]
        got = host(p.output(layer, pi))[tokens][:, rows]
        assert_close(got, ref, what=f"prefill M={p.m} layer {layer} {name}")


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
    last = CHECK_LAYERS[-1]
    outs = [prefill_pass.output(last, pi) for pi in range(len(synthetic.LAYER_PROJECTIONS))]
    first = [host(y).copy() for y in outs]
    for y in outs:
        y.fill_(7.0)
    prefill_pass.run()
    torch.cuda.synchronize()
    for pi, (a, y) in enumerate(zip(first, outs)):
        assert np.array_equal(a.view(np.uint16), host(y).view(np.uint16)), pi


def test_gate_up_run_as_one_gemm(prefill_pass):
    """The pass packs each layer's gate and up weights back to back and runs
    them as one GEMM: the per-projection outputs are views of one buffer."""
    assert all(f is not None for f in prefill_pass.fused)
    g = prefill_pass.output(0, 2)
    u = prefill_pass.output(0, 3)
    assert g.data_ptr() == prefill_pass.y_gate_up.data_ptr()
    assert u.data_ptr() == prefill_pass.y_gate_up.data_ptr() + g.shape[1] * 2
