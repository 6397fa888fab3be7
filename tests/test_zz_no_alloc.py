"""q4_gemv_skinny_noalloc (the entry point for callers that cannot allocate)
against q4_gemv_skinny, through the C ABI.

The two run the same plan and kernels, so their outputs must be bit-identical;
both are also held to the oracle's bar.  Two calls in a row share the static
scratch, the second with a smaller input, so the second must not see the
first's split-K state.
"""

import numpy as np
import pytest

from gpu_util import assert_close, dev, host, torch_cuda
from oracle import q4
from bit_quantized_weight_amd import gemv, gemv_noalloc, gemv_ws_bytes, pack, synthetic
from bit_quantized_weight_amd.binding import NOALLOC_SCRATCH_BYTES

pytestmark = pytest.mark.gpu

# (M, N, K, split_k): the speculative verify down-projection at M = 5 (the
# 4x4x4 kernel, 17 slices), then a smaller split-K shape (v_dot2 kernel, 3
# forced slices, ragged last row tile), then an M = 16 one (16x16x32 kernel).
CASES = [(5, 5120, 17408, 0), (3, 2000, 8192, 3), (16, 900, 4096, 0)]


def _case(torch, m, n, k, split_k, seed):
    w = synthetic.weights_device(n, k, seed)
    rows = np.unique(np.concatenate([[0, n - 1], np.random.default_rng(seed).integers(0, n, 48)]))
    wr = w.index_select(0, torch.as_tensor(rows, device="cuda")).cpu().numpy()
    codes, scales = pack(w)
    del w
    q, d = q4.quantize(wr)
    xh = synthetic.activations(m, k, seed + 1)
    return codes, scales, rows, q4.matmul(xh, q, d), dev(xh, torch)


def test_noalloc_matches_skinny_on_consecutive_calls():
    torch = torch_cuda()
    for i, (m, n, k, split_k) in enumerate(CASES):
        need = gemv_ws_bytes(m, n, k, split_k)
        assert 0 < need <= NOALLOC_SCRATCH_BYTES, (m, n, k, need)
        codes, scales, rows, ref, x = _case(torch, m, n, k, split_k, 4000 + 10 * i)
        y_ws = gemv(x, codes, scales, split_k=split_k)
        y_na = torch.full((m, n), 7.0, dtype=torch.float16, device="cuda")
        gemv_noalloc(x, codes, scales, y_na, split_k=split_k)
        torch.cuda.synchronize()
        a, b = host(y_ws), host(y_na)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), (m, n, k)
        assert_close(b[:, rows], ref, what=f"noalloc M={m} N={n} K={k}")


def test_noalloc_repeat_and_no_split():
    """A one-slice plan (no scratch used) and a repeat of a split plan."""
    torch = torch_cuda()
    codes, scales, rows, ref, x = _case(torch, 1, 4096, 5120, 0, 4100)
    assert gemv_ws_bytes(1, 4096, 5120, 0) == 0
    y = torch.empty((1, 4096), dtype=torch.float16, device="cuda")
    gemv_noalloc(x, codes, scales, y)
    torch.cuda.synchronize()
    assert_close(host(y)[:, rows], ref, what="noalloc one slice")
    assert np.array_equal(host(y).view(np.uint16), host(gemv(x, codes, scales)).view(np.uint16))
    codes, scales, rows, ref, x = _case(torch, 4, 3000, 17408, 0, 4200)
    outs = []
    for _ in range(2):
        y = torch.empty((4, 3000), dtype=torch.float16, device="cuda")
        gemv_noalloc(x, codes, scales, y)
        torch.cuda.synchronize()
        outs.append(host(y))
    assert np.array_equal(outs[0].view(np.uint16), outs[1].view(np.uint16))
    assert_close(outs[1][:, rows], ref, what="noalloc repeat")
