"""Oracle for the 4-bit block weight format and the skinny (M <= 8) matmul.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source passage: page 3 ("Qwen3.8-27B at 256K on a 24GB RTX PRO 4000 SFF"),
the paragraph saying decode streams quantized weights on every step and the
paragraph naming the Q4_0 GGUF.  The page does not define the format, so
the following plainest reading is used throughout (each step is a plain
definition, written out, with no blocking or reordering beyond it):

  * W is [N, K] (output-major, like a linear layer); Y = X . What^T.
  * Blocks are 32 consecutive weights along K, the reduction axis, so a block
    scale factors out of the dot product.
  * Scale: d32 = fl32(absmax / 7) (IEEE fp32 division), d = fp16_RNE(d32).
  * Codes use the stored fp16 scale: q = clamp(round_half_away(fl32(w / d)),
    -8, 7); an all-zero block (d == 0) has every code 0.
  * Packing: code k of a row goes to byte k // 2; even k in the low nibble,
    odd k in the high nibble, two's complement.  Codes [N, K/2] and scales
    [N, K/32] are separate planes.
  * Dequantization: what[n, k] = q[n, k] * d[n, k // 32], exact in float64.

Parity for the float matmul is pinned by brute force with exact rationals,
the all-ones closed form and one-hot activations (tests/test_oracle_q4.py).
"""

import numpy as np

BLOCK = 32          # weights per block along K
QMIN, QMAX = -8, 7  # signed 4-bit code range


def _round_half_away(v32):
    """Round fp32 values to integers, ties away from zero.

    Done in float64 on the exact fp32 value: floor(|v| + 0.5) is exact there,
    which avoids the fp32 trap where 0.49999997 + 0.5 rounds up to 1.
    """
    v = np.asarray(v32, dtype=np.float32).astype(np.float64)
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def block_scales(w):
    """fp16 block scales d[n, b] = fp16_RNE(fl32(absmax_b / 7)).

    ``w`` is float32 [N, K] with K % 32 == 0.
    """
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 32")
    amax = np.max(np.abs(w.reshape(n, k // BLOCK, BLOCK)), axis=2)
    d32 = amax / np.float32(7.0)              # IEEE fp32 division
    return d32.astype(np.float16)             # round to nearest even


def quantize(w):
    """Quantize float32 W [N, K] -> (codes int8 [N, K] in [-8, 7], d fp16 [N, K/32])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    d = block_scales(w)
    blocks = w.reshape(n, k // BLOCK, BLOCK)
    d32 = d.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = blocks / d32                      # fp32 quotient against the stored scale
    r = np.clip(_round_half_away(v), QMIN, QMAX)
    r[np.broadcast_to(d[:, :, None] == 0, r.shape)] = 0.0
    return r.astype(np.int8).reshape(n, k), d


def pack(q):
    """Pack int8 codes [N, K] (values in [-8, 7]) into bytes [N, K/2].

    Even k -> low nibble, odd k -> high nibble, two's complement.
    """
    q = np.asarray(q)
    if q.shape[1] % 2:
        raise ValueError("K must be even")
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def unpack(codes):
    """Inverse of ``pack``: bytes [N, K/2] -> int8 codes [N, K]."""
    c = np.asarray(codes, dtype=np.uint8)
    lo = (c & 0xF).astype(np.int16)
    hi = (c >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty((c.shape[0], c.shape[1] * 2), dtype=np.int8)
    out[:, 0::2] = lo
    out[:, 1::2] = hi
    return out


def dequantize(q, d):
    """what[n, k] = q[n, k] * d[n, k // 32] in float64 (exact)."""
    q = np.asarray(q, dtype=np.float64)
    d64 = np.asarray(d, dtype=np.float16).astype(np.float64)
    return q * np.repeat(d64, BLOCK, axis=1)


def matmul(x, q, d):
    """Skinny-route result Y[m, n] = sum_k x[m, k] * what[n, k] in float64.

    ``x`` is fp16 [M, K]; the GPU returns fp16(fp32 accumulation), the oracle
    is left unrounded.  Written as the plain definition: dequantize, then one
    float64 matrix product.
    """
    x64 = np.asarray(x, dtype=np.float16).astype(np.float64)
    return x64 @ dequantize(q, d).T


def matmul_blockwise(x, q, d):
    """Same result as ``matmul`` summed block by block: sum_b d[:, b] * (x_b . q_b^T).

    A second, independently arranged form of the definition; the two must
    agree to float64 rounding.
    """
    x64 = np.asarray(x, dtype=np.float16).astype(np.float64)
    q64 = np.asarray(q, dtype=np.float64)
    d64 = np.asarray(d, dtype=np.float16).astype(np.float64)
    m, k = x64.shape
    y = np.zeros((m, q64.shape[0]))
    for b in range(k // BLOCK):
        sl = slice(b * BLOCK, (b + 1) * BLOCK)
        y += (x64[:, sl] @ q64[:, sl].T) * d64[:, b][None, :]
    return y
