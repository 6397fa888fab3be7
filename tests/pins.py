"""Independent checks that pin the oracle to the mathematics, not to itself.

Everything here is exact-rational arithmetic with Python's ``fractions``:
correct rounding to binary32 / binary16 is implemented from the IEEE-754
definition (round to nearest, ties to even, gradual underflow), so none of
the oracle's NumPy casts or divisions is re-used.  Each ``pin_*`` function
takes the functions under test as arguments so that the mutant tests can
feed deliberately broken versions through the same checks.
"""

from fractions import Fraction
import math

import numpy as np

F32 = (24, -126)   # significand bits, minimum normal exponent
F16 = (11, -14)


def rne(fr, fmt):
    """Round an exact rational to the nearest value of a binary format (ties to even)."""
    p, emin = fmt
    fr = Fraction(fr)
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # now 2**e <= a < 2**(e+1)
    e = max(e, emin)
    ulp = Fraction(2) ** (e - p + 1)
    n = a / ulp
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def round_half_away(fr):
    fr = Fraction(fr)
    r = math.floor(abs(fr) + Fraction(1, 2))
    return r if fr >= 0 else -r


def exact_scale(block_values, divisor):
    """fp16_RNE(fl32(absmax / divisor)) as an exact rational (weights: divisor 7)."""
    a = max(abs(Fraction(float(v))) for v in block_values)
    return rne(rne(a / divisor, F32), F16)


def exact_code(w, d, lo, hi):
    """clamp(round_half_away(fl32(w / d)), lo, hi) with d the stored scale; 0 if d == 0."""
    if d == 0:
        return 0
    v = rne(Fraction(float(w)) / d, F32)
    return max(lo, min(hi, round_half_away(v)))


# --------------------------------------------------------------------------
# Weight quantizer pins
# --------------------------------------------------------------------------

def pin_scales(quantize, w):
    """Every stored scale equals the exact-rational rule."""
    w = np.asarray(w, np.float32)
    _, d = quantize(w)
    n, k = w.shape
    for i in range(n):
        for b in range(k // 32):
            want = exact_scale(w[i, 32 * b:32 * b + 32], 7)
            got = Fraction(float(d[i, b]))
            assert got == want, f"scale mismatch at row {i} block {b}: {got} vs {want}"


def pin_codes(quantize, w):
    """Every code equals the exact-rational rule, and is the nearest code to w/d
    except where the fp32 quotient itself crossed a rounding boundary."""
    w = np.asarray(w, np.float32)
    q, d = quantize(w)
    n, k = w.shape
    for i in range(n):
        for j in range(k):
            ds = Fraction(float(d[i, j // 32]))
            want = exact_code(w[i, j], ds, -8, 7)
            assert int(q[i, j]) == want, f"code mismatch at ({i},{j}): {q[i, j]} vs {want}"
            if ds != 0:
                t = Fraction(float(w[i, j])) / ds
                best = min(range(-8, 8), key=lambda c: (abs(t - c), -abs(c)))
                if best != want:
                    # allowed only when the exact quotient sits within one fp32 ulp of a tie
                    frac = abs(t) - math.floor(abs(t))
                    assert abs(frac - Fraction(1, 2)) <= abs(t) * Fraction(1, 2 ** 23), (i, j)


def pin_idempotent(quantize, dequant, w):
    """Q(deq(Q(W))) == Q(W): 7*d is exact in fp32 and fp16(fl32(7d/7)) == d."""
    q, d = quantize(np.asarray(w, np.float32))
    w2 = dequant(q, d).astype(np.float32)
    q2, d2 = quantize(w2)
    assert np.array_equal(d.view(np.uint16), d2.view(np.uint16))
    assert np.array_equal(q, q2)


def pin_error_bound(quantize, dequant, w):
    """|w - what| <= d/2 (up to one fp32 quotient rounding) for unclamped normal-scale blocks."""
    w = np.asarray(w, np.float32)
    q, d = quantize(w)
    wh = dequant(q, d)
    d64 = np.repeat(d.astype(np.float64), 32, axis=1)
    normal = d64 >= 2.0 ** -14
    err = np.abs(w.astype(np.float64) - wh)
    assert np.all(err[normal] <= d64[normal] * (0.5 + 2.0 ** -20))


# --------------------------------------------------------------------------
# Packing pins
# --------------------------------------------------------------------------

# Hand-derived: codes (1, -1, 7, -8, 0, 3, -5, 2) -> nibbles 1, F, 7, 8, 0, 3, B, 2;
# even k goes to the low nibble: bytes 0xF1, 0x87, 0x30, 0x2B.
HAND_CODES = [1, -1, 7, -8, 0, 3, -5, 2]
HAND_BYTES = [0xF1, 0x87, 0x30, 0x2B]


def pin_pack_literal(pack):
    got = np.asarray(pack(np.array([HAND_CODES], np.int8)), np.uint8).ravel().tolist()
    assert got == HAND_BYTES, got


def pin_roundtrip(pack, unpack):
    allb = np.arange(256, dtype=np.uint8).reshape(1, 256)
    assert np.array_equal(pack(unpack(allb)), allb)
    pairs = np.array([[a, b] for a in range(-8, 8) for b in range(-8, 8)], np.int8).reshape(1, -1)
    assert np.array_equal(unpack(pack(pairs)), pairs)


# --------------------------------------------------------------------------
# Matmul pins
# --------------------------------------------------------------------------

def exact_matmul(x, q, d):
    """Sum of exact rational products x[m,k] * q[n,k] * d[n,k//32]."""
    x = np.asarray(x, np.float16)
    m, k = x.shape
    n = q.shape[0]
    out = [[Fraction(0)] * n for _ in range(m)]
    for a in range(m):
        xs = [Fraction(float(v)) for v in x[a]]
        for c in range(n):
            s = Fraction(0)
            for j in range(k):
                s += xs[j] * int(q[c, j]) * Fraction(float(d[c, j // 32]))
            out[a][c] = s
    return out


def pin_matmul_exact(matmul, x, q, d, rel=1e-12):
    y = np.asarray(matmul(x, q, d), np.float64)
    ex = exact_matmul(x, q, d)
    scale = max(1e-300, max(abs(float(v)) for row in ex for v in row))
    for a in range(len(ex)):
        for c in range(len(ex[0])):
            assert abs(y[a, c] - float(ex[a][c])) <= rel * scale, (a, c, y[a, c], float(ex[a][c]))


def pin_one_hot(matmul, q, d):
    """x = e_k gives y[n] = q[n,k] * d[n, k//32] exactly."""
    n, k = q.shape
    for j in range(k):
        x = np.zeros((1, k), np.float16)
        x[0, j] = 1.0
        y = np.asarray(matmul(x, q, d), np.float64)[0]
        want = q[:, j].astype(np.float64) * d[:, j // 32].astype(np.float64)
        assert np.array_equal(y, want), j


# --------------------------------------------------------------------------
# A8 pins
# --------------------------------------------------------------------------

def pin_act_quant(quantize_act, x):
    x = np.asarray(x, np.float16)
    qa, sa = quantize_act(x)
    m, k = x.shape
    for i in range(m):
        for g in range(k // 64):
            blk = x[i, 64 * g:64 * g + 64]
            a = max(abs(Fraction(float(v))) for v in blk)
            s = rne(a / 127, F32)
            assert Fraction(float(sa[i, g])) == s, (i, g)
            for j in range(64):
                want = exact_code(blk[j], s, -127, 127)
                assert int(qa[i, 64 * g + j]) == want, (i, g, j)


def pin_block_sums(block_sums, qa, q):
    got = np.asarray(block_sums(qa, q))
    m, k = qa.shape
    n = q.shape[0]
    for i in range(m):
        for c in range(n):
            for b in range(k // 32):
                s = sum(int(qa[i, j]) * int(q[c, j]) for j in range(32 * b, 32 * b + 32))
                assert int(got[i, c, b]) == s, (i, c, b)


def pin_a8_exact(a8_matmul, qa, sa, q, d, rel=1e-12):
    y = np.asarray(a8_matmul(qa, sa, q, d), np.float64)
    m, k = qa.shape
    n = q.shape[0]
    ex = []
    for i in range(m):
        row = []
        for c in range(n):
            s = Fraction(0)
            for b in range(k // 32):
                ib = sum(int(qa[i, j]) * int(q[c, j]) for j in range(32 * b, 32 * b + 32))
                s += Fraction(float(sa[i, b // 2])) * Fraction(float(d[c, b])) * ib
            row.append(s)
        ex.append(row)
    scale = max(1e-300, max(abs(float(v)) for r in ex for v in r))
    for i in range(m):
        for c in range(n):
            assert abs(y[i, c] - float(ex[i][c])) <= rel * scale, (i, c)
