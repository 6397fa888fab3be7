"""q4_attn_decode on the GPU against the attention-read oracle.

The cache is what q4_pack makes of K and V rows (the weight format), the
queries are the last M positions (target token + drafts), and the geometry
is the reading used for the pages' model (page 3, "Qwen3.8-27B at 256K on a
24GB RTX PRO 4000 SFF", architecture paragraph): head dimension 256, 20
query heads, 4 K/V heads, plus other groupings.  Bar: max |o - oracle| <=
1e-2 RMS(oracle) per checked tensor.
"""

import numpy as np
import pytest

from gpu_util import assert_close, dev, host, torch_cuda
from oracle import attn
from bit_quantized_weight_amd import attn_decode, pack, synthetic

pytestmark = pytest.mark.gpu

D = 256


def _cache(torch, t, hkv, seed, std=1.0):
    """fp32 rows [T, H_kv * D] drawn on the device and packed; returns the
    device codes/scales and host copies."""
    w = synthetic.weights_device(t, hkv * D, seed, std=std)
    codes, scales = pack(w)
    del w
    return codes, scales, host(codes), host(scales)


def _run(torch, q, kc, ks, vc, vs, hkv):
    o = attn_decode(dev(q, torch), kc, ks, vc, vs, hkv)
    torch.cuda.synchronize()
    return host(o)


# (M, H_q, H_kv, T): the reading's geometry at M = 1..5 with ragged and short
# caches; MQA (one K/V head); R = M * G = 32 (the widest); T = M.  The query
# rows of a K/V head run in tiles of 16: R = 16 fills one tile, R = 17 puts a
# single row in a second.  T = 40,001 gives 64 key slices of 20 tiles with a
# one-key last tile.
SHAPES = [
    (1, 20, 4, 100), (5, 20, 4, 300), (4, 20, 4, 1000), (2, 20, 4, 33), (3, 20, 4, 3),
    (4, 8, 2, 777), (3, 4, 1, 65), (1, 32, 1, 4096), (1, 1, 1, 1), (6, 10, 2, 5000),
    (1, 17, 1, 500), (3, 20, 4, 40001),
]


@pytest.mark.parametrize("m,hq,hkv,t", SHAPES)
def test_attention_vs_oracle(m, hq, hkv, t):
    torch = torch_cuda()
    kc, ks, kch, ksh = _cache(torch, t, hkv, 100 + t)
    vc, vs, vch, vsh = _cache(torch, t, hkv, 200 + t)
    q = synthetic.activations(m * hq, D, 300 + t).reshape(m, hq, D)
    o = _run(torch, q, kc, ks, vc, vs, hkv)
    ref = attn.attention_decode(q, kch, ksh, vch, vsh, hkv)
    assert_close(o, ref, what=f"attn M={m} Hq={hq} Hkv={hkv} T={t}")
    o2 = _run(torch, q, kc, ks, vc, vs, hkv)
    assert np.array_equal(o.view(np.uint16), o2.view(np.uint16)), "not deterministic"


def test_peaked_scores():
    """Large queries (scores of several tens): nearly one-hot softmax rows,
    the regime where the running max and its rescaling matter."""
    torch = torch_cuda()
    m, hq, hkv, t = 2, 20, 4, 2000
    kc, ks, kch, ksh = _cache(torch, t, hkv, 11)
    vc, vs, vch, vsh = _cache(torch, t, hkv, 12)
    q = (synthetic.activations(m * hq, D, 13).astype(np.float32) * 6).astype(np.float16).reshape(m, hq, D)
    assert_close(_run(torch, q, kc, ks, vc, vs, hkv), attn.attention_decode(q, kch, ksh, vch, vsh, hkv),
                 what="peaked scores")


def test_constant_values_per_head():
    """V rows constant per K/V head: every query head returns its head's
    dequantized constant, whatever the weights (head grouping h // G)."""
    torch = torch_cuda()
    m, hq, hkv, t = 3, 20, 4, 500
    kc, ks, _, _ = _cache(torch, t, hkv, 21)
    vals = torch.tensor([0.5, -1.25, 2.0, 3.5], device="cuda").repeat_interleave(D)
    vc, vs = pack(vals[None, :].repeat(t, 1).contiguous())
    q = synthetic.activations(m * hq, D, 22).reshape(m, hq, D)
    o = _run(torch, q, kc, ks, vc, vs, hkv)
    ref = attn.attention_decode(q, host(kc), host(ks), host(vc), host(vs), hkv)
    for h in range(hq):
        want = ref[:, h, :]
        assert np.allclose(o[:, h, :].astype(np.float64), want, rtol=2e-3, atol=0), h


def test_causal_rows_past_the_limit_do_not_matter():
    """Query m sees rows 0 .. T - M + m: changing the rows it must not see
    leaves its output bit-identical."""
    torch = torch_cuda()
    m, hq, hkv, t = 5, 20, 4, 700
    kc, ks, _, _ = _cache(torch, t, hkv, 31)
    vc, vs, _, _ = _cache(torch, t, hkv, 32)
    q = synthetic.activations(m * hq, D, 33).reshape(m, hq, D)
    base = _run(torch, q, kc, ks, vc, vs, hkv)
    kc2, ks2, vc2, vs2 = kc.clone(), ks.clone(), vc.clone(), vs.clone()
    kc2[t - m + 1:] ^= 0x5A
    vc2[t - m + 1:] ^= 0xA5
    vs2[t - m + 1:] *= 3
    o = _run(torch, q, kc2, ks2, vc2, vs2, hkv)
    assert np.array_equal(o[0].view(np.uint16), base[0].view(np.uint16))
    assert not np.array_equal(o[m - 1].view(np.uint16), base[m - 1].view(np.uint16))


@pytest.mark.parametrize("m", [1, 5])
def test_full_context_sampled_heads(m):
    """The 256K-token context (T = 262,144, 64 slices of the keys): query
    heads of K/V heads 0 and 3 against the oracle run on those heads' columns
    of the cache (blocks never straddle heads, so a head's columns are a cache
    of their own)."""
    torch = torch_cuda()
    hq, hkv, t = 20, 4, 262144
    kc, ks, _, _ = _cache(torch, t, hkv, 41)
    vc, vs, _, _ = _cache(torch, t, hkv, 42)
    q = synthetic.activations(m * hq, D, 43 + m).reshape(m, hq, D)
    o = _run(torch, q, kc, ks, vc, vs, hkv)
    g_size = hq // hkv
    for g in (0, hkv - 1):
        cols, scols = slice(g * D // 2, (g + 1) * D // 2), slice(g * D // 32, (g + 1) * D // 32)
        heads = slice(g * g_size, (g + 1) * g_size)
        ref = attn.attention_decode(q[:, heads], host(kc[:, cols].contiguous()), host(ks[:, scols].contiguous()),
                                    host(vc[:, cols].contiguous()), host(vs[:, scols].contiguous()), 1)
        assert_close(o[:, heads], ref, what=f"attn T={t} M={m} kv head {g}")
