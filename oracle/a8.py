"""Oracle for the A8 prefill route (int8 activations x 4-bit block weights).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source passage: page 5 ("Qwen3.8-27B on RTX 4090: 5,000 tok/s Prefill
Reproduced"), section "Why the A8 artifact matters": for large prompt steps
the activations are quantized per token and per 64 channels and fed to an
int8 tensor-core matrix product against the groupwise weights.  The page
gives no scale form, rounding or clamp.  Readings used here, in the order the
route applies them (an encoding, so the steps are run as stated, not replaced
by a closed form):

  1. Activation groups are 64 consecutive channels along K of one token.
     sa[m, g] = fl32(absmax / 127) (IEEE fp32 division of the fp16 values
     widened to fp32).
  2. qa[m, k] = clamp(round_half_away(fl32(x / sa)), -127, 127); a zero group
     has sa = 0 and every qa = 0.
  3. The weight side is the same 32-element 4-bit blocks as the skinny route
     (codes sign-extended, no re-quantization); one activation group spans
     exactly two weight blocks.
  4. Block sums I[m, n, b] = sum_{k in b} qa[m, k] * q[n, k] are exact
     integers (|I| <= 32 * 127 * 8).
  5. Y[m, n] = sum_b sa[m, b // 2] * d[n, b] * I[m, n, b], here in float64
     (the GPU rescales in fp32 and rounds the result to fp16).
"""

import numpy as np

GROUP = 64   # activation channels per int8 scale
BLOCK = 32   # weights per 4-bit block


def _round_half_away(v32):
    v = np.asarray(v32, dtype=np.float32).astype(np.float64)
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


def quantize_act(x):
    """fp16 X [M, K] (K % 64 == 0) -> (qa int8 [M, K], sa float32 [M, K/64])."""
    x32 = np.asarray(x, dtype=np.float16).astype(np.float32)
    m, k = x32.shape
    if k % GROUP:
        raise ValueError("K must be a multiple of 64")
    g = x32.reshape(m, k // GROUP, GROUP)
    amax = np.max(np.abs(g), axis=2)
    sa = amax / np.float32(127.0)                       # IEEE fp32 division
    with np.errstate(divide="ignore", invalid="ignore"):
        v = g / sa[:, :, None]                          # fp32 quotient
    r = np.clip(_round_half_away(v), -127, 127)
    r[np.broadcast_to(sa[:, :, None] == 0, r.shape)] = 0.0
    return r.astype(np.int8).reshape(m, k), sa.astype(np.float32)


def block_sums(qa, q):
    """Exact integer block sums I[m, n, b] = sum_{k in b} qa[m, k] * q[n, k] (int64).

    Computed as one float64 product per block of 32: every partial sum is an
    integer far below 2**53, so the float64 result is exact.
    """
    qa64 = np.asarray(qa, dtype=np.float64)
    q64 = np.asarray(q, dtype=np.float64)
    m, k = qa64.shape
    n = q64.shape[0]
    out = np.empty((m, n, k // BLOCK), dtype=np.int64)
    for b in range(k // BLOCK):
        sl = slice(b * BLOCK, (b + 1) * BLOCK)
        out[:, :, b] = (qa64[:, sl] @ q64[:, sl].T).astype(np.int64)
    return out


def matmul(qa, sa, q, d):
    """A8 result Y[m, n] = sum_b sa[m, b//2] * d[n, b] * I[m, n, b] in float64.

    Loops over blocks so the [M, N, K/32] integer tensor is never held whole.
    """
    qa64 = np.asarray(qa, dtype=np.float64)
    q64 = np.asarray(q, dtype=np.float64)
    sa64 = np.asarray(sa, dtype=np.float32).astype(np.float64)
    d64 = np.asarray(d, dtype=np.float16).astype(np.float64)
    m, k = qa64.shape
    y = np.zeros((m, q64.shape[0]))
    for b in range(k // BLOCK):
        sl = slice(b * BLOCK, (b + 1) * BLOCK)
        ib = qa64[:, sl] @ q64[:, sl].T                 # exact integers
        y += (sa64[:, b // 2][:, None] * ib) * d64[:, b][None, :]
    return y


def prefill(x, q, d):
    """Whole A8 route from fp16 activations: quantize_act, then ``matmul``."""
    qa, sa = quantize_act(x)
    return matmul(qa, sa, q, d)
