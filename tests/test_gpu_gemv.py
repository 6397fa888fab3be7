"""q4_gemv_skinny on the GPU against the fp64 oracle (M = 1..16)."""

import functools

import numpy as np
import pytest

from gpu_util import assert_close, dev, host, torch_cuda
from oracle import q4
from bit_quantized_weight_amd import gemv, pack, synthetic

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=4)
def packed(n, k, seed):
    """Weights packed on the GPU plus the oracle's own quantization of them."""
    torch = torch_cuda()
    w = synthetic.weights(n, k, seed)
    codes, scales = pack(dev(w, torch))
    q, d = q4.quantize(w)
    return codes, scales, q, d


def run(x, codes, scales, split_k=0):
    torch = torch_cuda()
    y = gemv(dev(x, torch), codes, scales, split_k=split_k)
    torch.cuda.synchronize()
    return host(y)


def test_tiny_matvec():
    codes, scales, q, d = packed(512, 256, 0)
    x = synthetic.activations(1, 256, 1)
    assert_close(run(x, codes, scales), q4.matmul(x, q, d), what="tiny")


@pytest.mark.parametrize("m", range(1, 9))
@pytest.mark.parametrize("n,k", [(100, 96), (300, 1056), (64, 512), (257, 5120), (70, 8192)])
def test_shapes_and_ragged_tails(m, n, k):
    """Ragged N (not a multiple of the 64-row tile) and K (not a multiple of 512)."""
    codes, scales, q, d = packed(n, k, 10 + n)
    x = synthetic.activations(m, k, 20 + m)
    assert_close(run(x, codes, scales), q4.matmul(x, q, d), what=f"M={m} N={n} K={k}")


@pytest.mark.parametrize("split", [1, 2, 3, 7, 64])
@pytest.mark.parametrize("m", [3, 4, 6, 7])
def test_explicit_split_k(m, split):
    """The v_dot2 kernel (M = 3) and the 4x4x4 kernel with one (M = 4) and two
    (M = 6, 7) A operands with a forced slice count, over a ragged last row tile
    (N = 200)."""
    codes, scales, q, d = packed(200, 2048, 30)
    x = synthetic.activations(m, 2048, 31)
    ref = q4.matmul(x, q, d)
    y1 = run(x, codes, scales, split)
    assert_close(y1, ref, what=f"M={m} split={split}")
    y2 = run(x, codes, scales, split)
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16)), "split-K not deterministic"


@pytest.mark.parametrize("m", [5, 7])
@pytest.mark.parametrize("k", [2080, 5120, 8192])
def test_forced_one_slice_two_operands(m, k):
    """split_k = 1 with two A operands (M = 5, 7) on the 4x4x4 kernel: one
    slice of 5 steps (the 6-step copy), of 10 steps (the 10-step copy, the
    largest LDS use: 76.8 KB at M = 7), and K = 8192 capped at 10 steps (two
    slices).  Ragged last row tile (N = 200)."""
    codes, scales, q, d = packed(200, k, 96)
    x = synthetic.activations(m, k, 97 + m)
    ref = q4.matmul(x, q, d)
    y1 = run(x, codes, scales, 1)
    assert_close(y1, ref, what=f"M={m} K={k} split_k=1")
    assert np.array_equal(run(x, codes, scales, 1).view(np.uint16), y1.view(np.uint16))


@pytest.mark.parametrize("m,split", [(4, 2), (6, 2), (7, 3)])
def test_explicit_split_k_long_slices(m, split):
    """A forced small slice count on a tall K (544 blocks, 34 steps): at M = 4
    the slices are capped at 10 steps (4 slices), with two A operands at 6
    steps (6 slices), over a ragged last row tile and a ragged last step."""
    n, k = 1000, 17408 - 32
    rows = tuple(np.unique(np.concatenate([[0, 31, 32, n - 1],
                                           np.random.default_rng(m).integers(0, n, 40)])).tolist())
    codes, scales, q, d = packed_sampled(n, k, 94, rows)
    x = synthetic.activations(m, k, 95)
    y = run(x, codes, scales, split)
    assert_close(y[:, list(rows)], q4.matmul(x, q, d), what=f"M={m} split={split}")


@pytest.mark.parametrize("m", [8, 13])
def test_explicit_split_k_matrix_core(m):
    """16x16x32 kernel with many slices (K = 4096, split_k = 64 gives 32
    one-step slices): the fixup's partial loads go out in several chunks
    (18 slices per chunk at M = 8, 9 at M = 13), over a ragged last row tile."""
    codes, scales, q, d = packed(300, 4096, 40)
    x = synthetic.activations(m, 4096, 41 + m)
    ref = q4.matmul(x, q, d)
    y1 = run(x, codes, scales, 64)
    assert_close(y1, ref, what=f"M={m} split=64")
    y2 = run(x, codes, scales, 64)
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16)), "split-K not deterministic"
    y0 = run(x, codes, scales, 0)
    assert_close(y0, ref, what=f"M={m} split=auto")


def test_workspace_shared_across_shapes():
    """One workspace serving a split-K shape with few tiles, then one with many:
    the first call's partials must never be read as the second call's counters."""
    torch = torch_cuda()
    from bit_quantized_weight_amd import gemv_ws_bytes, q4_gemv_skinny_raw
    ca, sa_, qa, da = packed(200, 2048, 30)
    cb, sb, qb, db = packed(3000, 1024, 32)
    xa = synthetic.activations(8, 2048, 33)
    xb = synthetic.activations(2, 1024, 34)
    nbytes = max(gemv_ws_bytes(8, 200, 2048, 64), gemv_ws_bytes(2, 3000, 1024, 0))
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        ya = torch.empty((8, 200), dtype=torch.float16, device="cuda")
        q4_gemv_skinny_raw(dev(xa, torch), ca, sa_, ya, split_k=64, ws=ws)
        yb = torch.empty((2, 3000), dtype=torch.float16, device="cuda")
        q4_gemv_skinny_raw(dev(xb, torch), cb, sb, yb, split_k=0, ws=ws)
        torch.cuda.synchronize()
        assert_close(host(ya), q4.matmul(xa, qa, da), what="shape A")
        assert_close(host(yb), q4.matmul(xb, qb, db), what="shape B")


@pytest.mark.parametrize("m", [4, 6, 7, 8])
def test_one_hot_bit_exact(m):
    """x = e_k gives fp16(q[n,k] * d[n,k//32]): one product, rounded once
    (M = 4, 6, 7: the 4x4x4 kernel with one and two A operands; M = 8: the
    16x16x32 kernel)."""
    n, k = 96, 256
    codes, scales, q, d = packed(n, k, 40)
    for start in range(0, k, m):
        live = [r for r in range(m) if start + r < k]
        x = np.zeros((m, k), np.float16)
        for r in live:
            x[r, start + r] = 1.0
        y = run(x, codes, scales)
        for r in live:
            kk = start + r
            want = (q[:, kk].astype(np.float64) * d[:, kk // 32].astype(np.float64)).astype(np.float16)
            assert np.array_equal(y[r], want), kk


@pytest.mark.parametrize("k,y16", [(256, 256.0), (5120, 5120.0), (17408, 17408.0)])
def test_all_ones_closed_form(k, y16):
    """W = 1, x = 1: y = K (1 - 2**-12) exactly in fp32, which rounds to K in fp16."""
    torch = torch_cuda()
    codes, scales = pack(torch.ones((64, k), dtype=torch.float32, device="cuda"))
    for m in (1, 5):
        y = run(np.ones((m, k), np.float16), codes, scales)
        assert np.all(y == np.float16(y16)), (m, np.unique(y))


def test_decode_gate_up():
    """Decode GEMV, FFN gate/up shape: M = 1, K = 5120, N = 17408."""
    w = synthetic.WORKLOADS["decode_gate_up"]
    codes, scales, q, d = packed(w["N"], w["K"], synthetic.WEIGHT_SEED)
    x = synthetic.activations(1, w["K"], synthetic.ACT_SEED)
    assert_close(run(x, codes, scales), q4.matmul(x, q, d), what="decode_gate_up")


@pytest.mark.parametrize("n,k", [(5000, 17408), (2560, 17408 - 32), (8192, 8192 + 32)])
@pytest.mark.parametrize("m", [3, 4])
def test_split_row_tiles_4x4x4(m, n, k):
    """The 4x4x4 kernel's split forms at M = 3 and 4: 64-row tiles (N = 5000, 711
    workgroups: 79 tiles, the last one ragged, x 9 slices of 4 steps;
    N = 8192, K = 8224) and 32-row tiles (N = 2560, where 64-row tiles would
    give only 360 workgroups), each over a ragged last step where K is not a
    multiple of 512.  Sampled rows include both ends."""
    rows = tuple(np.unique(np.concatenate([[0, 63, 64, n - 65, n - 1],
                                           np.random.default_rng(n).integers(0, n, 60)])).tolist())
    codes, scales, q, d = packed_sampled(n, k, 92, rows)
    x = synthetic.activations(m, k, 93)
    y = run(x, codes, scales)
    assert_close(y[:, list(rows)], q4.matmul(x, q, d), what=f"M={m} K={k} N={n}")
    assert np.array_equal(run(x, codes, scales).view(np.uint16), y.view(np.uint16))


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5])
def test_verify_down(m):
    """Speculative verify, down-projection shape: K = 17408, N = 5120, M = 1..5."""
    w = synthetic.WORKLOADS["verify_down"]
    codes, scales, q, d = packed(w["N"], w["K"], synthetic.WEIGHT_SEED)
    x = synthetic.activations(m, w["K"], synthetic.ACT_SEED)
    assert_close(run(x, codes, scales), q4.matmul(x, q, d), what=f"verify_down M={m}")


def test_invariants_bit_exact():
    """Deterministic reduction: repeats are bit-identical and y(2x) = 2 y(x)
    exactly (every step scales exactly by a power of two) wherever y is an fp16
    normal.  Below 2^-14 the fp16 output is subnormal with spacing 2^-24, so
    2 fp16(y) sits on a grid twice as coarse as fp16(2y); there the two may
    differ by up to 1.5 * 2^-24.  y(-x) = -y(x) is checked to the tolerance
    only: the hardware fp16 dot product does not round symmetrically in sign,
    so negation can move a result by one fp16 ulp."""
    codes, scales, q, d = packed(5120, 17408, synthetic.WEIGHT_SEED)
    for m in (1, 2, 3, 4, 5, 6, 8):   # v_dot2, 4x4x4 (one and two A operands), 16x16x32
        x = synthetic.activations(m, 17408, 50)
        y = run(x, codes, scales)
        y2 = run((x.astype(np.float32) * 2).astype(np.float16), codes, scales)
        twice = (y.astype(np.float32) * 2).astype(np.float16)
        normal = np.abs(y.astype(np.float32)) >= 2.0 ** -14
        assert np.array_equal(y2[normal], twice[normal]), m
        gap = np.abs(y2[~normal].astype(np.float64) - twice[~normal].astype(np.float64))
        assert np.all(gap <= 1.5 * 2.0 ** -24), (m, gap.max())
        yn = run(-x, codes, scales)
        assert_close(-yn, q4.matmul(x, q, d), what=f"negated input M={m}")
        for _ in range(5):
            assert np.array_equal(run(x, codes, scales).view(np.uint16), y.view(np.uint16)), m


def test_permuted_rows_permute_outputs():
    codes, scales, q, d = packed(300, 1056, 60)
    x = synthetic.activations(2, 1056, 61)
    y = run(x, codes, scales)
    perm = np.random.default_rng(0).permutation(300)
    torch = torch_cuda()
    idx = torch.from_numpy(perm).cuda()
    yp = run(x, codes[idx].contiguous(), scales[idx].contiguous())
    assert np.array_equal(yp.view(np.uint16), y[:, perm].view(np.uint16))


def test_tiny_and_large_activations():
    """fp16-subnormal activations (row 0) and large magnitudes (row 2).

    Row 0's outputs are themselves fp16-subnormal (|y| ~ 1e-6, spacing 2^-24),
    so the bar there adds the output format's own rounding, half a spacing;
    rows 1 and 2 use the plain bar."""
    codes, scales, q, d = packed(128, 1024, 70)
    rng = np.random.default_rng(71)
    x = (rng.standard_normal((3, 1024)) * np.array([[1e-6], [1.0], [300.0]])).astype(np.float16)
    y = run(x, codes, scales)
    ref = q4.matmul(x, q, d)
    rms0 = np.sqrt(np.mean(ref[0] ** 2))
    assert np.max(np.abs(y[0].astype(np.float64) - ref[0])) <= 1e-2 * rms0 + 2.0 ** -25
    for r in (1, 2):
        assert_close(y[r:r + 1], ref[r:r + 1], what=f"row {r}")


def test_empty_shapes():
    torch = torch_cuda()
    codes, scales, q, d = packed(64, 256, 80)
    # K == 0: empty sum, zeros
    y = gemv(torch.zeros((2, 0), dtype=torch.float16, device="cuda"),
             torch.zeros((64, 0), dtype=torch.uint8, device="cuda"),
             torch.zeros((64, 0), dtype=torch.float16, device="cuda"))
    torch.cuda.synchronize()
    assert y.shape == (2, 64) and not host(y).any()
    # N == 0
    y = gemv(torch.ones((1, 256), dtype=torch.float16, device="cuda"),
             torch.zeros((0, 128), dtype=torch.uint8, device="cuda"),
             torch.zeros((0, 8), dtype=torch.float16, device="cuda"))
    assert y.shape == (1, 0)


@pytest.mark.parametrize("m", [1, 4, 8])
def test_large_n_split_counters(m):
    """N just under 2^19 with split-K: 65,535 row tiles of 8 rows at M = 1
    (16,384 of 32 rows at M = 4), so the arrival counters span the whole
    counter region at M = 1.  Sampled rows,
    including both ends, are checked against the oracle."""
    torch = torch_cuda()
    n, k = (1 << 19) - 8, 2048
    w = synthetic.weights_device(n, k, 77)
    rng = np.random.default_rng(78)
    rows = np.unique(np.concatenate([[0, 1, 131071, 131072, 262143, n - 2, n - 1],
                                     rng.integers(0, n, 40)]))
    wr = w.index_select(0, torch.as_tensor(rows, device="cuda")).cpu().numpy()
    codes, scales = pack(w)
    del w
    q, d = q4.quantize(wr)
    x = synthetic.activations(m, k, 79 + m)
    y = run(x, codes, scales, split_k=2)
    assert_close(y[:, rows], q4.matmul(x, q, d), what=f"N={n} M={m} split 2")


@pytest.mark.parametrize("m", [1, 5])
def test_max_k(m):
    """K at the entry point's limit (2^24, 524,288 blocks per row) over 40 rows:
    the longest rows the library accepts, split into many slices; the byte
    offsets of the last row's blocks and of the activations are the largest
    any kernel forms.  Sampled rows (both ends included) against the oracle."""
    torch = torch_cuda()
    n, k = 40, 1 << 24
    w = synthetic.weights_device(n, k, 87)
    rows = np.array([0, 17, n - 1])
    wr = w.index_select(0, torch.as_tensor(rows, device="cuda")).cpu().numpy()
    codes, scales = pack(w)
    del w
    q, d = q4.quantize(wr)
    x = synthetic.activations_device(m, k, 88 + m)
    y = gemv(x, codes, scales)
    torch.cuda.synchronize()
    assert_close(host(y)[:, rows], q4.matmul(host(x), q, d), what=f"M={m} N={n} K={k}")


@functools.lru_cache(maxsize=2)
def packed_sampled(n, k, seed, rows):
    """Weights generated and packed on the GPU; the oracle quantizes only the
    sampled rows (quantization is per row, so they match the full pack)."""
    torch = torch_cuda()
    w = synthetic.weights_device(n, k, seed)
    wr = w.index_select(0, torch.as_tensor(rows, device="cuda")).cpu().numpy()
    codes, scales = pack(w)
    del w
    q, d = q4.quantize(wr)
    return codes, scales, q, d


@pytest.mark.parametrize("k", [992, 4064, 5088, 6112, 7136, 9184, 11232, 12256])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_vector_kernel_slice_forms(m, k):
    """Every form of the M <= 4 kernels on one slice per row tile (N = 4100:
    257 tiles of 16 rows): K from 31 to 383 blocks, each with a ragged last
    step.  M <= 3 (the v_dot2 kernel, 32-block steps): the short no-refill
    form, the full-depth one and the refilled ring.  M = 4 (the 4x4x4
    kernel, 16-block steps): every depth up to 10 steps with one 4-row group
    per wave, and past 10 steps the split into slices with two groups per
    wave; M = 3 takes the same split form past 160 blocks."""
    n = 4100
    rows = tuple(np.unique(np.concatenate([[0, 15, 16, n - 1],
                                           np.random.default_rng(k).integers(0, n, 60)])).tolist())
    codes, scales, q, d = packed_sampled(n, k, 90, rows)
    x = synthetic.activations(m, k, 91 + m)
    y = run(x, codes, scales)
    assert_close(y[:, list(rows)], q4.matmul(x, q, d), what=f"M={m} K={k} N={n}")


BATCH_SHAPES = [(100, 96), (300, 1056), (257, 5120), (70, 8192), (5120, 17408), (64, 512)]


@pytest.mark.parametrize("m", [1, 3, 4, 5, 8, 13, 16])
def test_batched_matches_oracle_and_repeats(m):
    """One persistent launch over six matmuls of mixed, ragged shapes (K not
    a multiple of 128 included): each output within the bar of the oracle,
    and repeated runs of the plan bit-identical (fixed summation order)."""
    torch = torch_cuda()
    from bit_quantized_weight_amd import batched_plan
    items, refs = [], []
    for i, (n, k) in enumerate(BATCH_SHAPES):
        codes, scales, q, d = packed(n, k, 900 + i)
        x = synthetic.activations(m, k, 950 + i)
        y = torch.full((m, n), 7.0, dtype=torch.float16, device="cuda")
        items.append((dev(x, torch), codes, scales, y))
        refs.append(q4.matmul(x, q, d))
    batch = batched_plan(items)
    first = None
    for rep in range(3):
        for it in items:
            it[3].fill_(7.0)
        batch.run()
        torch.cuda.synchronize()
        outs = [host(it[3]).copy() for it in items]
        for (n, k), got, ref in zip(BATCH_SHAPES, outs, refs):
            assert_close(got, ref, what=f"batched M={m} N={n} K={k} rep {rep}")
        if first is None:
            first = outs
        else:
            for a, b in zip(first, outs):
                assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), m


def test_batched_aligned_and_ragged_k_variants():
    """A batch whose every K is a multiple of 128 takes the packed-scale
    kernel variant; adding one ragged K switches the whole batch to the
    other variant.  Both agree with the oracle."""
    torch = torch_cuda()
    from bit_quantized_weight_amd import batched_plan
    for shapes in ([(96, 1024), (300, 5120)], [(96, 1024), (300, 5120), (70, 1056)]):
        items, refs = [], []
        for i, (n, k) in enumerate(shapes):
            codes, scales, q, d = packed(n, k, 960 + i)
            x = synthetic.activations(5, k, 970 + i)
            items.append((dev(x, torch), codes, scales,
                          torch.empty((5, n), dtype=torch.float16, device="cuda")))
            refs.append(q4.matmul(x, q, d))
        batch = batched_plan(items)
        assert batch.plan.variant == (1 if len(shapes) == 2 else 0)
        batch.run()
        torch.cuda.synchronize()
        for (n, k), it, ref in zip(shapes, items, refs):
            assert_close(host(it[3]), ref, what=f"variant test N={n} K={k}")


@pytest.mark.parametrize("m", [9, 12, 13, 16])
@pytest.mark.parametrize("n,k", [(100, 96), (300, 1056), (257, 5120), (70, 8192)])
def test_wide_verify_shapes(m, n, k):
    """Verify widths 9..16 (a 12-token draft window verifies 13 rows) on
    ragged shapes: N not a multiple of the 64-row tile, K not a multiple of
    the slice."""
    codes, scales, q, d = packed(n, k, 10 + n)
    x = synthetic.activations(m, k, 20 + m)
    assert_close(run(x, codes, scales), q4.matmul(x, q, d), what=f"M={m} N={n} K={k}")


@pytest.mark.parametrize("m", [8, 13, 16])
def test_verify_down_wide(m):
    """Speculative verify, down-projection shape, at M = 8, 13, 16."""
    w = synthetic.WORKLOADS["verify_down"]
    codes, scales, q, d = packed(w["N"], w["K"], synthetic.WEIGHT_SEED)
    x = synthetic.activations(m, w["K"], synthetic.ACT_SEED)
    assert_close(run(x, codes, scales), q4.matmul(x, q, d), what=f"verify_down M={m}")


def test_one_hot_bit_exact_wide():
    """One-hot rows through the 16-row matrix-core path: every output is one
    product rounded once, so the result is bit-exact."""
    n, k = 96, 256
    codes, scales, q, d = packed(n, k, 41)
    for start in (0, 16, 240):
        x = np.zeros((16, k), np.float16)
        for r in range(16):
            x[r, start + r] = 1.0
        y = run(x, codes, scales)
        for r in range(16):
            kk = start + r
            want = (q[:, kk].astype(np.float64) * d[:, kk // 32].astype(np.float64)).astype(np.float16)
            assert np.array_equal(y[r], want), kk


def test_binding_rejects_short_workspace_and_bad_output():
    """The binding passes the caller's whole workspace size, so a workspace
    one byte short of what the plan needs is rejected by the library
    (WORKSPACE) before anything is enqueued; a y of the wrong shape or dtype
    is rejected by the binding."""
    torch = torch_cuda()
    from bit_quantized_weight_amd import Q4WError, gemv_ws_bytes, q4_gemv_skinny_raw
    codes, scales, q, d = packed(200, 2048, 30)
    x = dev(synthetic.activations(4, 2048, 31), torch)
    need = gemv_ws_bytes(4, 200, 2048, 3)
    assert need > 0
    short = torch.zeros(need - 1, dtype=torch.uint8, device="cuda")
    y = torch.empty((4, 200), dtype=torch.float16, device="cuda")
    with pytest.raises(Q4WError) as e:
        q4_gemv_skinny_raw(x, codes, scales, y, split_k=3, ws=short)
    assert e.value.status == -4
    with pytest.raises(ValueError):
        q4_gemv_skinny_raw(x, codes, scales, torch.empty((4, 199), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        q4_gemv_skinny_raw(x, codes, scales, torch.empty((4, 200), dtype=torch.float32, device="cuda"))
    ok = torch.zeros(need, dtype=torch.uint8, device="cuda")
    q4_gemv_skinny_raw(x, codes, scales, y, split_k=3, ws=ok)
    torch.cuda.synchronize()
    assert_close(host(y), q4.matmul(synthetic.activations(4, 2048, 31), q, d), what="exact workspace")


def test_workspace_cache_is_per_stream():
    """Calls on two streams get two cached workspaces (their split-K state
    must not be shared), calls on one stream share one."""
    torch = torch_cuda()
    from bit_quantized_weight_amd import binding
    codes, scales, q, d = packed(200, 2048, 30)
    xh = synthetic.activations(4, 2048, 31)
    x = dev(xh, torch)
    ref = q4.matmul(xh, q, d)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    ys = []
    for s in (s1, s2, s1):
        with torch.cuda.stream(s):
            ys.append(gemv(x, codes, scales, split_k=3))
    torch.cuda.synchronize()
    keys = [k for k in binding._ws_cache if k[0] == "gemv"]
    streams = {k[2] for k in keys}
    assert s1.cuda_stream in streams and s2.cuda_stream in streams
    for y in ys:
        assert_close(host(y), ref, what="per-stream workspace")
