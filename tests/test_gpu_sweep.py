"""Seeded random shapes for every route, against the oracles.

The shape lists are drawn once from fixed seeds (so every run checks the same
cases) over the ranges each entry point accepts: any M of the skinny route,
ragged N and K, the A8 route's token counts and widths around its tile forms,
and the attention read's groupings and cache lengths.  The same bars as the
targeted tests: fp16 outputs within 1e-2 x RMS of the oracle, A8 int32 block
sums bit-exact.
"""

import numpy as np
import pytest

from gpu_util import assert_close, dev, host, torch_cuda
from oracle import a8, attn, q4
from bit_quantized_weight_amd import a8w4_debug_block_acc, a8w4_gemm, attn_decode, gemv, pack, synthetic

pytestmark = pytest.mark.gpu


def _skinny_shapes(count=24, seed=2024):
    rs = np.random.RandomState(seed)
    out = []
    while len(out) < count:
        m = int(rs.randint(1, 17))
        n = int(rs.randint(1, 6001))
        k = 32 * int(rs.randint(1, 401))
        if n * k <= 16 << 20:
            out.append((m, n, k))
    return out


def _a8_shapes(count=12, seed=2025):
    rs = np.random.RandomState(seed)
    out = []
    while len(out) < count:
        m = int(rs.randint(1, 301))
        n = int(rs.randint(1, 1501))
        k = 64 * int(rs.randint(1, 81))
        if m * n * k <= 1 << 30:
            out.append((m, n, k))
    return out


def _attn_shapes(count=8, seed=2026):
    rs = np.random.RandomState(seed)
    out = []
    while len(out) < count:
        m = int(rs.randint(1, 7))
        hkv = int(rs.choice([1, 2, 4]))
        g = int(rs.randint(1, 32 // m + 1))
        t = int(rs.randint(m, 3001))
        out.append((m, g * hkv, hkv, t))
    return out


@pytest.mark.parametrize("m,n,k", _skinny_shapes())
def test_skinny_random_shapes(m, n, k):
    torch = torch_cuda()
    w = synthetic.weights(n, k, n + k)
    codes, scales = pack(dev(w, torch))
    q, d = q4.quantize(w)
    x = synthetic.activations(m, k, m + n)
    y = gemv(dev(x, torch), codes, scales)
    torch.cuda.synchronize()
    assert_close(host(y), q4.matmul(x, q, d), what=f"skinny M={m} N={n} K={k}")


@pytest.mark.parametrize("m,n,k", _a8_shapes())
def test_a8_random_shapes(m, n, k):
    torch = torch_cuda()
    w = synthetic.weights(n, k, 3 * n + k)
    codes, scales = pack(dev(w, torch))
    q, d = q4.quantize(w)
    x = synthetic.activations(m, k, m + 7 * n)
    acc = a8w4_debug_block_acc(dev(x, torch), codes, scales)
    y = a8w4_gemm(dev(x, torch), codes, scales)
    torch.cuda.synchronize()
    qa, _ = a8.quantize_act(x)
    assert np.array_equal(host(acc), a8.block_sums(qa, q).astype(np.int32)), f"A8 block sums M={m} N={n} K={k}"
    assert_close(host(y), a8.prefill(x, q, d), what=f"A8 M={m} N={n} K={k}")


@pytest.mark.parametrize("m,hq,hkv,t", _attn_shapes())
def test_attention_random_shapes(m, hq, hkv, t):
    torch = torch_cuda()
    D = 256
    k_rows = synthetic.weights(t, hkv * D, 5 * t + hkv, std=1.0)
    v_rows = synthetic.weights(t, hkv * D, 7 * t + hkv, std=1.0)
    kc, ks = pack(dev(k_rows, torch))
    vc, vs = pack(dev(v_rows, torch))
    qh = synthetic.activations(m * hq, D, 11 * t + m).reshape(m, hq, D)
    o = attn_decode(dev(qh, torch), kc, ks, vc, vs, hkv)
    torch.cuda.synchronize()
    ref = attn.attention_decode(qh, host(kc), host(ks), host(vc), host(vs), hkv)
    assert_close(host(o), ref, what=f"attn M={m} Hq={hq} Hkv={hkv} T={t}")
