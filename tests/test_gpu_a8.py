"""A8 prefill route on the GPU: int8 codes/scales and int32 block sums bit-exact,
rescaled fp16 output within the bar of the A8 oracle."""

import numpy as np
import pytest

from gpu_util import assert_close, dev, host, torch_cuda
from oracle import a8, q4
from bit_quantized_weight_amd import (a8_quantize_act, a8w4_debug_block_acc, a8w4_gemm, pack,
                                      synthetic)
from test_oracle_a8 import _special_acts

pytestmark = pytest.mark.gpu


def _packed(n, k, seed):
    torch = torch_cuda()
    w = synthetic.weights(n, k, seed)
    codes, scales = pack(dev(w, torch))
    q, d = q4.quantize(w)
    return codes, scales, q, d


@pytest.mark.parametrize("m,k", [(1, 64), (37, 256), (256, 5120), (5, 17408)])
def test_act_quant_bit_exact(m, k):
    torch = torch_cuda()
    x = synthetic.activations(m, k, 100 + m)
    xq, sa = a8_quantize_act(dev(x, torch))
    torch.cuda.synchronize()
    qa, sa_ref = a8.quantize_act(x)
    assert np.array_equal(host(xq), qa)
    assert np.array_equal(host(sa).view(np.uint32), sa_ref.view(np.uint32))


def test_act_quant_special():
    torch = torch_cuda()
    x = _special_acts()
    xq, sa = a8_quantize_act(dev(x, torch))
    torch.cuda.synchronize()
    qa, sa_ref = a8.quantize_act(x)
    assert np.array_equal(host(xq), qa)
    assert np.array_equal(host(sa).view(np.uint32), sa_ref.view(np.uint32))


def _every_fp16_value(absmax):
    """Rows of one 64-channel group: channel 0 holds absmax (so every group's
    scale is sa = fl32(absmax / 127)), channels 1..63 run through every finite
    fp16 value of magnitude at most absmax, both signs."""
    a = np.float16(absmax)
    pos = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)
    vals = pos[pos <= a]
    vals = np.concatenate([vals, -vals])
    n = -(-len(vals) // 63)
    flat = np.zeros(n * 63, np.float16)
    flat[:len(vals)] = vals
    x = np.zeros((n, 64), np.float16)
    x[:, 0] = a
    x[:, 1:] = flat.reshape(n, 63)
    return x


@pytest.mark.parametrize("absmax", [127.0, 100.0, 37.5, 3.0, 0.001, 65504.0])
def test_act_quant_every_fp16_value(absmax):
    """Every fp16 activation against a fixed group scale: each value whose
    quotient x / sa falls at or next to a rounding tie is met, so the
    quantizers' fast path and its exact fallback are both checked, bit-exact
    against the oracle (row-major quantizer directly; the GEMM's tiled
    quantizer through the int32 block sums)."""
    torch = torch_cuda()
    x = _every_fp16_value(absmax)
    xq, sa = a8_quantize_act(dev(x, torch))
    torch.cuda.synchronize()
    qa, sa_ref = a8.quantize_act(x)
    assert np.array_equal(host(xq), qa)
    assert np.array_equal(host(sa).view(np.uint32), sa_ref.view(np.uint32))
    codes, scales, q, d = _packed(16, 64, 250)
    acc = a8w4_debug_block_acc(dev(x, torch), codes, scales)
    torch.cuda.synchronize()
    assert np.array_equal(host(acc), a8.block_sums(qa, q).astype(np.int32))


@pytest.mark.parametrize("m,n,k", [(1, 32, 64), (31, 48, 256), (33, 130, 128), (128, 128, 512),
                                   (130, 257, 192), (256, 512, 5120)])
def test_block_sums_bit_exact(m, n, k):
    """Exact int32 block sums from the matrix-core kernel's debug epilogue."""
    torch = torch_cuda()
    codes, scales, q, d = _packed(n, k, 200 + n)
    x = synthetic.activations(m, k, 300 + m)
    acc = a8w4_debug_block_acc(dev(x, torch), codes, scales)
    torch.cuda.synchronize()
    qa, _ = a8.quantize_act(x)
    assert np.array_equal(host(acc), a8.block_sums(qa, q).astype(np.int32))


def test_block_sums_extremes():
    """|I| = 32 * 127 * 8 = 32512 at the extremes of both code ranges."""
    torch = torch_cuda()
    w = np.full((32, 64), -8.0, np.float32)
    w[:, 0] = 7.0                                       # absmax 8 ... codes: 7 at k=0
    codes, scales = pack(dev(w, torch))
    q, d = q4.quantize(w)
    x = np.full((32, 64), -1.0, np.float16)
    acc = a8w4_debug_block_acc(dev(x, torch), codes, scales)
    torch.cuda.synchronize()
    qa, _ = a8.quantize_act(x)
    assert np.array_equal(host(acc), a8.block_sums(qa, q).astype(np.int32))


@pytest.mark.parametrize("m,n,k", [(1, 32, 64), (31, 48, 256), (130, 257, 192), (256, 512, 5120),
                                   (64, 256, 17408)])
def test_a8_gemm_vs_oracle(m, n, k):
    torch = torch_cuda()
    codes, scales, q, d = _packed(n, k, 400 + n)
    x = synthetic.activations(m, k, 500 + m)
    y = a8w4_gemm(dev(x, torch), codes, scales)
    torch.cuda.synchronize()
    assert_close(host(y), a8.prefill(x, q, d), what=f"A8 M={m} N={n} K={k}")


@pytest.mark.parametrize("n", [16000, 16500])
def test_tile_forms_block_sums_and_gemm(n):
    """Both workgroup tile forms at M = 130 (two 128-row tiles): N = 16000 gives
    250 tiles of 128 x 128, below one per CU, so the 64-row form runs (with a
    half-empty and an empty 64-row tile); N = 16500 gives 258 and the 128-row
    form runs, with a ragged last column tile.  Block sums bit-exact, result
    against the A8 oracle."""
    torch = torch_cuda()
    m, k = 130, 192
    codes, scales, q, d = _packed(n, k, 800 + n)
    x = synthetic.activations(m, k, 801)
    acc = a8w4_debug_block_acc(dev(x, torch), codes, scales)
    y = a8w4_gemm(dev(x, torch), codes, scales)
    torch.cuda.synchronize()
    qa, _ = a8.quantize_act(x)
    assert np.array_equal(host(acc), a8.block_sums(qa, q).astype(np.int32))
    assert_close(host(y), a8.prefill(x, q, d), what=f"A8 M={m} N={n} K={k}")


@pytest.mark.parametrize("n,k", [(38400, 256), (38477, 256), (38400, 192)])
def test_chunk_balanced_form(n, k):
    """M = 256: 600 (or 602, with a ragged last column tile) tiles of 128 x 128
    make more than one round of the 512 resident workgroups, so the
    chunk-balanced form runs: 512 equal ranges of 3 chunks (2 per tile), and
    most tiles are summed by two workgroups.  K = 192 has a half chunk at the
    end of every tile.  Against the A8 oracle, and a second call
    bit-identical to the first."""
    torch = torch_cuda()
    m = 256
    codes, scales, q, d = _packed(n, k, 900 + n)
    x = synthetic.activations(m, k, 901)
    xd = dev(x, torch)
    y1 = host(a8w4_gemm(xd, codes, scales))
    y2 = host(a8w4_gemm(xd, codes, scales))
    torch.cuda.synchronize()
    assert_close(y1, a8.prefill(x, q, d), what=f"A8 M={m} N={n} K={k}")
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


def test_chunk_balanced_form_block_sums():
    """The exact int32 block sums from the chunk-balanced form: M = 256,
    N = 38400 (600 tiles of 128 x 128 over 512 workgroups, so chunk ranges
    cut tiles), K = 192 (a half chunk at the end of every tile).  Every block
    of a tile is computed by exactly one workgroup, which writes it.  Checked
    bit-exactly on sampled columns of every column tile, all tokens."""
    torch = torch_cuda()
    m, n, k = 256, 38400, 192
    codes, scales, q, d = _packed(n, k, 910)
    x = synthetic.activations(m, k, 911)
    acc = a8w4_debug_block_acc(dev(x, torch), codes, scales)
    rng = np.random.default_rng(912)
    cols = np.unique(np.concatenate([np.arange(0, n, 128), np.arange(127, n, 128),
                                     rng.integers(0, n, 600)]))
    got = host(acc.index_select(1, torch.as_tensor(cols, device=acc.device)))
    del acc
    qa, _ = a8.quantize_act(x)
    assert np.array_equal(got, a8.block_sums(qa, q[cols]).astype(np.int32))


def test_prepare_then_gemm_matches_one_call():
    """Quantize once, reuse for two weight matrices; bit-identical to the one-call route."""
    torch = torch_cuda()
    from bit_quantized_weight_amd import a8w4_gemm_prepared, a8w4_prepare
    k = 1024
    c1, s1, q1, d1 = _packed(96, k, 700)
    c2, s2, q2, d2 = _packed(160, k, 701)
    x = dev(synthetic.activations(70, k, 702), torch)
    ws = a8w4_prepare(x)
    y1 = a8w4_gemm_prepared(ws, 70, k, c1, s1)
    y2 = a8w4_gemm_prepared(ws, 70, k, c2, s2)
    r1 = a8w4_gemm(x, c1, s1)
    r2 = a8w4_gemm(x, c2, s2)
    torch.cuda.synchronize()
    assert np.array_equal(host(y1).view(np.uint16), host(r1).view(np.uint16))
    assert np.array_equal(host(y2).view(np.uint16), host(r2).view(np.uint16))


def test_a8_all_ones():
    torch = torch_cuda()
    k = 5120
    codes, scales = pack(torch.ones((64, k), dtype=torch.float32, device="cuda"))
    y = a8w4_gemm(torch.ones((40, k), dtype=torch.float16, device="cuda"), codes, scales)
    torch.cuda.synchronize()
    assert np.all(host(y) == np.float16(5120.0))


def test_prefill_full_size_sampled():
    """The A8 prefill GEMM at M = 2048, K = 5120, N = 17408 (the launch the
    benchmark times); every column of 24 sampled token rows checked."""
    torch = torch_cuda()
    wl = synthetic.WORKLOADS["prefill_a8"]
    M, K, N = wl["M"], wl["K"], wl["N"]
    codes, scales, q, d = _packed(N, K, synthetic.WEIGHT_SEED)
    x = synthetic.activations(M, K, synthetic.ACT_SEED)
    y = a8w4_gemm(dev(x, torch), codes, scales)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 127, 128, 1023, M - 1],
                                     np.random.default_rng(7).integers(0, M, 16)]))
    yh = host(y)[rows]
    ref = a8.prefill(x[rows], q, d)
    assert_close(yh, ref, what="prefill_a8 sampled rows")


def test_a8_empty_shapes():
    torch = torch_cuda()
    codes, scales, q, d = _packed(32, 128, 600)
    y = a8w4_gemm(torch.zeros((0, 128), dtype=torch.float16, device="cuda"), codes, scales)
    assert y.shape == (0, 32)
    y = a8w4_gemm(torch.zeros((3, 0), dtype=torch.float16, device="cuda"),
                  torch.zeros((32, 0), dtype=torch.uint8, device="cuda"),
                  torch.zeros((32, 0), dtype=torch.float16, device="cuda"))
    torch.cuda.synchronize()
    assert y.shape == (3, 32) and not host(y).any()


def test_act_quant_in_pieces():
    """a8_quantize_act launches rows in pieces of at most 2^25 groups: at
    K = 5120 (80 groups per row) a piece is 419,430 rows, so 419,500 rows (a
    4.3 GB input) take two launches.  Rows on both sides of the split and the
    last row are bit-exact against the oracle."""
    torch = torch_cuda()
    m, k = 419_500, 5120
    x = synthetic.activations_device(m, k, 123)
    xq, sa = a8_quantize_act(x)
    torch.cuda.synchronize()
    rows = [0, 419_429, 419_430, 419_431, m - 1]
    sel = torch.as_tensor(rows, device="cuda")
    xr = x.index_select(0, sel).cpu().numpy()
    xqr = xq.index_select(0, sel).cpu().numpy()
    sar = sa.index_select(0, sel).cpu().numpy()
    del x, xq, sa
    qa, sa_ref = a8.quantize_act(xr)
    assert np.array_equal(xqr, qa)
    assert np.array_equal(sar.view(np.uint32), sa_ref.view(np.uint32))


def test_a8_zero_k_fill_in_pieces():
    """K = 0 fills y with zeros in pieces of at most 2^28 elements: y of
    1024 x 262,208 (268,500,992 elements, first filled with ones) ends all zero."""
    torch = torch_cuda()
    m, n = 1024, (1 << 18) + 64
    y = torch.ones((m, n), dtype=torch.float16, device="cuda")
    a8w4_gemm(torch.zeros((m, 0), dtype=torch.float16, device="cuda"),
              torch.zeros((n, 0), dtype=torch.uint8, device="cuda"),
              torch.zeros((n, 0), dtype=torch.float16, device="cuda"), y=y)
    torch.cuda.synchronize()
    assert not bool((y != 0).any())
