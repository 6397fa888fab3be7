"""Exact pins of the skinny kernels on the GPU, for every kernel and form.

Layout pin (one-hot activations): x = e_k in row r gives y[r, n] =
fp16(q[n, k] * d[n, k // 32]).  Inside the kernels every other product is an
exact zero, the unpack bias cancels exactly, and q * d is exact in fp32, so
the only rounding is the final fp16 store: the result is bit-exact.  A
mistake in nibble order, block or scale indexing, slice offsets, the split-K
fixup or the row mapping changes some output.

Closed form (all ones): W = 1 quantizes to d = fp16(1/7), q = 7, so
What = 1 - 2**-12 and y = K (1 - 2**-12), which is exact in fp32 and rounds
to K in fp16 for the K used here.

The 4-bit format follows the reading of the Q4_0 weights named on page 3
("Qwen3.8-27B at 256K on a 24GB RTX PRO 4000 SFF"): 32-weight blocks, an
fp16 scale absmax / 7 and signed 4-bit codes.
"""

import numpy as np
import pytest

from gpu_util import dev, host, torch_cuda
from oracle import q4
from bit_quantized_weight_amd import batched_plan, gemv, pack, synthetic

pytestmark = pytest.mark.gpu

N_SMALL = 40     # three row tiles of 16 rows, the last one ragged


def one_hot_positions(k, seed, splits=(2, 3)):
    """Positions that touch every nibble slot of a block, both ends of K, the
    neighbourhood of every 512-weight step boundary and of the slice
    boundaries of small forced splits, plus a few random ones."""
    nb = k // 32
    pos = set(range(min(64, k)))
    pos.update(range(max(0, k - 48), k))
    for s in range(512, k, 512):
        pos.update((s - 1, s, s + 1))
    for S in splits:
        bps = -(-nb // S)
        for j in range(1, S):
            pos.update((32 * bps * j - 1, 32 * bps * j))
    pos.update(np.random.default_rng(seed).integers(0, k, 24).tolist())
    return sorted(p for p in pos if 0 <= p < k)


def expected_one_hot(w_cols, k):
    """fp16(q[:, k] * d[:, k // 32]) from the oracle's quantization of the
    32-weight column block holding k (quantization is per row and block, so
    one column block gives the same codes and scale as the whole matrix)."""
    q, d = q4.quantize(w_cols)
    return (q[:, k % 32].astype(np.float64) * d[:, 0].astype(np.float64)).astype(np.float16)


def check_one_hot(torch, w_dev, codes, scales, m, k, split_k, seed):
    n = codes.shape[0]
    positions = one_hot_positions(k, seed)
    blocks = {}
    for start in range(0, len(positions), m):
        live = positions[start:start + m]
        x = np.zeros((m, k), np.float16)
        for r, kk in enumerate(live):
            x[r, kk] = 1.0
        y = host(gemv(dev(x, torch), codes, scales, split_k=split_k))
        for r, kk in enumerate(live):
            b = kk // 32
            if b not in blocks:
                blocks[b] = w_dev[:, 32 * b:32 * b + 32].cpu().numpy()
            want = expected_one_hot(blocks[b], kk)
            assert y.shape == (m, n)
            assert np.array_equal(y[r], want), f"M={m} K={k} split_k={split_k} position {kk}"
        # rows past the live ones (last call) hold zero activations: y = 0
        for r in range(len(live), m):
            assert not y[r].any(), f"M={m} K={k} zero row {r}"


# (M, K, split_k): every form of the v_dot2 kernel (M <= 3) and of the 4x4x4
# kernel with two A operands (M = 5), on N = 40 rows.
#   M = 1, 2:  K = 4064 one slice of 4 steps (short copy); 6112 one slice of
#              6 steps (full ring, no refill); 8224 one slice of 9 steps (the
#              refilled ring); 8224 split in 3 (slices of 3 steps); M = 1,
#              K = 16384 split_k = 1: two ring-refilled slices of 12 steps
#              (a forced slice count raised to fit the LDS budget).
#   M = 3:     4064 short; 5120 one slice of 5 steps; 8224 split_k = 1, two
#              slices (capped at 160 blocks); 8224 split in 3; 8224 auto (the
#              4x4x4 kernel's split form with two row groups).
#   M = 5:     2080 split_k = 1 (one slice, the 6-step copy); 5120 split_k = 1
#              (one slice, the 10-step copy); 8192 split_k = 1 (capped at
#              10 steps: two slices); 5120 auto (4-step slices, two row
#              groups); 5120 split in 3.
FORMS = [
    (1, 4064, 1), (1, 6112, 1), (1, 8224, 1), (1, 8224, 3), (1, 16384, 1),
    (2, 4064, 1), (2, 6112, 1), (2, 8224, 1), (2, 8224, 3),
    (3, 4064, 1), (3, 5120, 1), (3, 8224, 1), (3, 8224, 3), (3, 8224, 0),
    (5, 2080, 1), (5, 5120, 1), (5, 8192, 1), (5, 5120, 0), (5, 5120, 3),
]


@pytest.mark.parametrize("m,k,split_k", FORMS)
def test_one_hot_every_form(m, k, split_k):
    torch = torch_cuda()
    w = synthetic.weights_device(N_SMALL, k, 500 + k)
    codes, scales = pack(w)
    check_one_hot(torch, w, codes, scales, m, k, split_k, seed=k + m)


@pytest.mark.parametrize("m,n,k", [(1, 4100, 5120), (4, 8192, 8192)])
def test_one_hot_default_plans_wide(m, n, k):
    """The default plans at realistic widths: M = 1 on 257 row tiles (one
    slice, no split); M = 4 on the 4x4x4 kernel's 64-row tiles (four row
    groups per wave, 4-step slices, 512 workgroups)."""
    torch = torch_cuda()
    w = synthetic.weights_device(n, k, 600 + m)
    codes, scales = pack(w)
    check_one_hot(torch, w, codes, scales, m, k, 0, seed=n)


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6, 7, 8, 16])
def test_all_ones_every_route(m):
    """W = 1, x = 1 through the route each M takes (v_dot2, 4x4x4 with one or
    two A operands, 16x16x32), one slice and split."""
    torch = torch_cuda()
    for k in (5120, 17408):
        codes, scales = pack(torch.ones((64, k), dtype=torch.float32, device="cuda"))
        for split_k in (0, 1, 3):
            y = host(gemv(torch.ones((m, k), dtype=torch.float16, device="cuda"), codes, scales,
                          split_k=split_k))
            assert np.all(y == np.float16(k)), (m, k, split_k, np.unique(y))


@pytest.mark.parametrize("m", [1, 5, 16])
@pytest.mark.parametrize("shapes", [
    [(100, 96), (300, 1056), (257, 5120), (70, 8192)],    # ragged K: the 2-byte-scale variant
    [(96, 1024), (300, 5120), (64, 8192)],                # K % 128 == 0: the packed-scale variant
], ids=["ragged", "aligned"])
def test_batched_one_hot(m, shapes):
    """The persistent streaming kernel: one plan over several matmuls, run
    again for every set of one-hot positions (the plan reads x at run time).
    Every output of every matmul is one product rounded once."""
    torch = torch_cuda()
    mats = []
    for i, (n, k) in enumerate(shapes):
        w = synthetic.weights_device(n, k, 700 + i)
        codes, scales = pack(w)
        x = torch.zeros((m, k), dtype=torch.float16, device="cuda")
        y = torch.empty((m, n), dtype=torch.float16, device="cuda")
        mats.append(dict(w=w, codes=codes, scales=scales, x=x, y=y, k=k,
                         pos=one_hot_positions(k, 800 + i, splits=())))
    batch = batched_plan([(t["x"], t["codes"], t["scales"], t["y"]) for t in mats])
    assert batch.plan.variant == (1 if shapes[0] == (96, 1024) else 0)
    rounds = max(-(-len(t["pos"]) // m) for t in mats)
    cache = {}
    for rnd in range(rounds):
        live = []
        for t in mats:
            ps = t["pos"][rnd * m:(rnd + 1) * m]
            xh = np.zeros((m, t["k"]), np.float16)
            for r, kk in enumerate(ps):
                xh[r, kk] = 1.0
            t["x"].copy_(torch.from_numpy(xh))
            t["y"].fill_(7.0)
            live.append(ps)
        batch.run()
        torch.cuda.synchronize()
        for i, (t, ps) in enumerate(zip(mats, live)):
            y = host(t["y"])
            for r, kk in enumerate(ps):
                key = (i, kk // 32)
                if key not in cache:
                    cache[key] = t["w"][:, 32 * (kk // 32):32 * (kk // 32) + 32].cpu().numpy()
                want = expected_one_hot(cache[key], kk)
                assert np.array_equal(y[r], want), f"batched M={m} matmul {i} position {kk}"
            for r in range(len(ps), m):
                assert not y[r].any(), f"batched M={m} matmul {i} zero row {r}"


@pytest.mark.parametrize("m", [1, 5, 16])
def test_batched_all_ones(m):
    """All-ones closed form through the streaming kernel: y = K exactly."""
    torch = torch_cuda()
    ks = (256, 5120, 17408, 1056)
    items = []
    for k in ks:
        codes, scales = pack(torch.ones((64, k), dtype=torch.float32, device="cuda"))
        items.append((torch.ones((m, k), dtype=torch.float16, device="cuda"), codes, scales,
                      torch.zeros((m, 64), dtype=torch.float16, device="cuda")))
    batch = batched_plan(items)
    batch.run()
    torch.cuda.synchronize()
    for k, it in zip(ks, items):
        y = host(it[3])
        assert np.all(y == np.float16(k)), (m, k, np.unique(y))
