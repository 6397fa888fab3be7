"""Pins of the attention-read oracle (oracle/attn.py) to the mathematics.

Each pin takes the function under test as an argument, so the planted
mistakes in tests/test_oracle_mutants.py run through the same checks.  None
of them re-types the oracle's formula:

  * constant V rows per K/V head: any set of softmax weights averages a
    constant to itself, so o equals that head's dequantized value (the
    scale computed with exact rationals) -- pins the head grouping and the
    normalization;
  * q = 0: every score is 0, the weights are uniform, so o is the plain
    mean of the visible V rows -- pins the causal visible length;
  * two positions: p0 = (1 + tanh((s0 - s1) / 2)) / 2, the logistic form of
    a two-way softmax, with s = q . k / sqrt(D) from exactly dequantized
    one-hot rows -- pins the score scale;
  * one dominant score (scores near +-4096, so an exp without the max
    subtracted overflows): o is that position's V row;
  * causality: rows a query must not see can change without changing its
    output, the last row it sees cannot;
  * permutation: the last query sees every row, and the result does not
    depend on their order.

Page 3 ("Qwen3.8-27B at 256K on a 24GB RTX PRO 4000 SFF"), architecture and
bandwidth paragraphs: the 16 full-attention layers read a 4-bit K/V cache.
"""

import math
from fractions import Fraction

import numpy as np

import pins
from oracle import attn, q4


def make_cache(w):
    """Quantize fp32 rows [T, H*D] into the cache layout (codes, scales)."""
    q, d = q4.quantize(np.asarray(w, np.float32))
    return q4.pack(q), d


def rand_cache(t, h, d, seed):
    rng = np.random.default_rng(seed)
    return make_cache(rng.standard_normal((t, h * d)).astype(np.float32))


def rand_q(m, hq, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((m, hq, d)) * scale).astype(np.float16)


# ---- pins -----------------------------------------------------------------

def pin_constant_v(fn, m=3, hq=8, hkv=2, d=64, t=40):
    """V rows constant per head g (value c_g = (g + 1) / 2): o[m, h, :] equals
    7 * fp16(c_g / 7), the exact dequantized constant of head h // (hq / hkv)."""
    kc, ks = rand_cache(t, hkv, d, 1)
    c = [(g + 1) / 2 for g in range(hkv)]
    vw = np.concatenate([np.full((t, d), cg, np.float32) for cg in c], axis=1)
    vc, vs = make_cache(vw)
    o = fn(rand_q(m, hq, d, 2), kc, ks, vc, vs, hkv)
    group = hq // hkv
    for h in range(hq):
        dq = pins.exact_scale([c[h // group]] * 32, 7)
        want = float(7 * dq)
        assert np.allclose(o[:, h, :], want, rtol=0, atol=1e-12 * want), h


def pin_uniform(fn, m=4, hq=4, hkv=2, d=64, t=9):
    """q = 0: o[m, h] is the mean of V rows 0 .. T - M + m of head h // G."""
    kc, ks = rand_cache(t, hkv, d, 3)
    vc, vs = rand_cache(t, hkv, d, 4)
    v = q4.dequantize(q4.unpack(vc), vs).reshape(t, hkv, d)
    o = fn(np.zeros((m, hq, d), np.float16), kc, ks, vc, vs, hkv)
    group = hq // hkv
    for mi in range(m):
        n_vis = t - m + mi + 1
        for h in range(hq):
            want = np.mean(v[:n_vis, h // group, :], axis=0)
            assert np.allclose(o[mi, h], want, rtol=0, atol=1e-12), (mi, h)


def pin_two_positions(fn, d=256):
    """T = 2, one query: keys one-hot along channel 0 with values +k0 and -k1
    (each quantizes to code +-7 and scale fp16(|k| / 7)), q = a e_0.  Then
    s_t = a K[t, 0] / sqrt(D) and p0 = (1 + tanh((s0 - s1) / 2)) / 2."""
    k0, k1, a = 1.75, 0.625, 12.0
    kw = np.zeros((2, d), np.float32)
    kw[0, 0], kw[1, 0] = k0, -k1
    kc, ks = make_cache(kw)
    rng = np.random.default_rng(5)
    vc, vs = make_cache(rng.standard_normal((2, d)).astype(np.float32))
    v = q4.dequantize(q4.unpack(vc), vs)
    q = np.zeros((1, 1, d), np.float16)
    q[0, 0, 0] = a
    o = fn(q, kc, ks, vc, vs, 1)
    s0 = a * 7 * float(pins.exact_scale([k0], 7)) / math.sqrt(d)
    s1 = -a * 7 * float(pins.exact_scale([k1], 7)) / math.sqrt(d)
    p0 = (1 + math.tanh((s0 - s1) / 2)) / 2
    want = p0 * v[0] + (1 - p0) * v[1]
    assert np.allclose(o[0, 0], want, rtol=0, atol=1e-12), (o[0, 0, :4], want[:4])


def pin_dominant(fn, d=64, t=12, star=7):
    """Scores near +-4096: one position carries all the weight, so o is its
    V row (an exp without the max subtracted overflows here)."""
    kw = np.zeros((t, d), np.float32)
    kw[:, 0] = -1.0
    kw[star, 0] = 1.0
    kc, ks = make_cache(kw)
    vc, vs = rand_cache(t, 1, d, 6)
    v = q4.dequantize(q4.unpack(vc), vs)
    q = np.zeros((1, 1, d), np.float16)
    q[0, 0, 0] = 32768.0                 # s = +-32768 * 7 fp16(1/7) / 8, about +-4096
    o = fn(q, kc, ks, vc, vs, 1)
    assert np.all(np.isfinite(o))
    assert np.allclose(o[0, 0], v[star], rtol=0, atol=1e-12)


def pin_causal(fn, m=4, hq=2, hkv=1, d=32, t=10):
    """Query mi sees rows 0 .. t - m + mi: rows past that may change freely,
    the last visible one may not."""
    kw = np.random.default_rng(7).standard_normal((t, hkv * d)).astype(np.float32)
    vw = np.random.default_rng(8).standard_normal((t, hkv * d)).astype(np.float32)
    q = rand_q(m, hq, d, 9)
    base = fn(q, *make_cache(kw), *make_cache(vw), hkv)
    for mi in range(m - 1):
        last = t - m + mi
        kw2, vw2 = kw.copy(), vw.copy()
        kw2[last + 1:] = -kw2[last + 1:] * 3
        vw2[last + 1:] = vw2[last + 1:] + 5
        o2 = fn(q, *make_cache(kw2), *make_cache(vw2), hkv)
        assert np.array_equal(o2[mi], base[mi]), mi
        vw3 = vw.copy()
        vw3[last] += 4
        o3 = fn(q, *make_cache(kw), *make_cache(vw3), hkv)
        assert not np.allclose(o3[mi], base[mi]), mi


def pin_permutation(fn, hq=4, hkv=2, d=64, t=16):
    """One query sees every row: permuting the rows leaves o unchanged."""
    kw = np.random.default_rng(10).standard_normal((t, hkv * d)).astype(np.float32)
    vw = np.random.default_rng(11).standard_normal((t, hkv * d)).astype(np.float32)
    q = rand_q(1, hq, d, 12, scale=2.0)
    perm = np.random.default_rng(13).permutation(t)
    a = fn(q, *make_cache(kw), *make_cache(vw), hkv)
    b = fn(q, *make_cache(kw[perm]), *make_cache(vw[perm]), hkv)
    assert np.allclose(a, b, rtol=0, atol=1e-12)


ALL_PINS = [pin_constant_v, pin_uniform, pin_two_positions, pin_dominant, pin_causal, pin_permutation]


# ---- the oracle against its pins ------------------------------------------

def test_constant_v():
    pin_constant_v(attn.attention_decode)


def test_uniform_scores():
    pin_uniform(attn.attention_decode)


def test_two_positions_closed_form():
    pin_two_positions(attn.attention_decode)


def test_dominant_position():
    pin_dominant(attn.attention_decode)


def test_causal_visibility():
    pin_causal(attn.attention_decode)


def test_permutation_invariance():
    pin_permutation(attn.attention_decode)


def test_cache_is_the_weight_format():
    """The cache layout is the weight quantizer's output on the K rows: the
    dequantized cache reshaped per head equals q * d for each 32-block."""
    t, h, d = 5, 2, 64
    w = np.random.default_rng(14).standard_normal((t, h * d)).astype(np.float32)
    codes, scales = make_cache(w)
    k = attn.dequantize_cache(codes, scales, h)
    qc, dc = q4.quantize(w)
    for ti in range(t):
        for hi in range(h):
            for b in range(d // 32):
                blk = k[ti, hi, 32 * b:32 * b + 32]
                col = hi * d + 32 * b
                exact = [Fraction(int(c)) * Fraction(float(dc[ti, col // 32])) for c in qc[ti, col:col + 32]]
                assert [Fraction(float(v)) for v in blk] == exact
