"""Full 64-layer decode-step weight pass at M = 5 (speculative verify of 1 + 4
drafted tokens): sampled output rows of sampled layers against the oracle,
and HIP-graph replays bit-identical to the eager pass."""

import numpy as np
import pytest

from gpu_util import assert_close, host, torch_cuda
from oracle import q4
from bit_quantized_weight_amd import synthetic
from bit_quantized_weight_amd.decode import DecodeStep

pytestmark = pytest.mark.gpu

M = 5
CHECK_LAYERS = (0, 31, 63)


def _rows(n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, 30)]))


@pytest.fixture(scope="module")
def step():
    torch = torch_cuda()
    keep = {}
    for layer in CHECK_LAYERS:
        for pi, (_, k, n) in enumerate(synthetic.LAYER_PROJECTIONS):
            keep[(layer, pi)] = _rows(n, 10 * layer + pi)
    s = DecodeStep(M, keep_rows=keep)
    s.run()
    torch.cuda.synchronize()
    yield s
    del s
    torch.cuda.empty_cache()


def test_decode_step_sampled_rows(step):
    xs = [host(x) for x in step.xs]
    for layer in CHECK_LAYERS:
        for pi, (name, k, n) in enumerate(synthetic.LAYER_PROJECTIONS):
            rows = _rows(n, 10 * layer + pi)
            q, d = q4.quantize(step.kept[(layer, pi)])
            ref = q4.matmul(xs[pi], q, d)                      # [M, len(rows)]
            got = host(step.ys[layer][pi])[:, rows]
            assert_close(got, ref, what=f"layer {layer} {name}")


def test_decode_step_graph_replay_matches_eager(step):
    torch = torch_cuda()
    eager = [[host(y).copy() for y in ys] for ys in step.ys]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step.run()
    for rep in range(3):
        for ys in step.ys:                 # poison the outputs between replays
            for y in ys:
                y.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for layer in (0, 17, 63):
            for pi in range(len(synthetic.LAYER_PROJECTIONS)):
                assert np.array_equal(host(step.ys[layer][pi]).view(np.uint16),
                                      eager[layer][pi].view(np.uint16)), (rep, layer, pi)


def test_decode_step_batched(step):
    """The whole step as one persistent launch: sampled rows of three layers
    against the oracle, then three graph replays of the batched launch, each
    bit-identical to the first batched run."""
    torch = torch_cuda()
    step.plan_batched()
    for ys in step.ys:
        for y in ys:
            y.fill_(7.0)
    step.run_batched()
    torch.cuda.synchronize()
    xs = [host(x) for x in step.xs]
    for layer in CHECK_LAYERS:
        for pi, (name, k, n) in enumerate(synthetic.LAYER_PROJECTIONS):
            rows = _rows(n, 10 * layer + pi)
            q, d = q4.quantize(step.kept[(layer, pi)])
            assert_close(host(step.ys[layer][pi])[:, rows], q4.matmul(xs[pi], q, d),
                         what=f"batched layer {layer} {name}")
    first = {(l, pi): host(step.ys[l][pi]).copy() for l in (0, 17, 63)
             for pi in range(len(synthetic.LAYER_PROJECTIONS))}
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step.run_batched()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step.run_batched()
    for rep in range(3):
        for ys in step.ys:
            for y in ys:
                y.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (l, pi), ref in first.items():
            assert np.array_equal(host(step.ys[l][pi]).view(np.uint16), ref.view(np.uint16)), (rep, l, pi)
