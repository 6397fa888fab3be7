"""Planted mistakes: each broken copy of an oracle function must fail a pin.

This shows the pins are strong enough to catch the plausible slips (a wrong
rounding rule, a wrong divisor, a swapped nibble, a transposed operand, a
dropped block, a wrong group index).  The mistakes live only in this file,
on the CPU; the oracle itself is untouched.
"""

import numpy as np
import pytest

import pins
from oracle import a8, q4
from bit_quantized_weight_amd import synthetic

from test_oracle_q4 import _special_rows
from test_oracle_a8 import _special_acts


def _w():
    return np.concatenate([synthetic.weights(4, 64, seed=51), _special_rows()])


# ---- weight quantizer mutants -------------------------------------------

def quantize_half_even(w):
    w = np.asarray(w, np.float32)
    n, k = w.shape
    d = q4.block_scales(w)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = w.reshape(n, k // 32, 32) / d.astype(np.float32)[:, :, None]
        r = np.clip(np.rint(v.astype(np.float64)), -8, 7)
    r[np.broadcast_to(d[:, :, None] == 0, r.shape)] = 0
    return r.astype(np.int8).reshape(n, k), d


def quantize_div8(w):
    w = np.asarray(w, np.float32)
    n, k = w.shape
    a = np.max(np.abs(w.reshape(n, k // 32, 32)), axis=2)
    d = (a / np.float32(8.0)).astype(np.float16)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = w.reshape(n, k // 32, 32) / d.astype(np.float32)[:, :, None]
        r = np.clip(np.sign(v) * np.floor(np.abs(v.astype(np.float64)) + 0.5), -8, 7)
    r[np.broadcast_to(d[:, :, None] == 0, r.shape)] = 0
    return r.astype(np.int8).reshape(n, k), d


def quantize_fp32_scale(w):
    """Codes from the unrounded fp32 scale instead of the stored fp16 one."""
    w = np.asarray(w, np.float32)
    n, k = w.shape
    a = np.max(np.abs(w.reshape(n, k // 32, 32)), axis=2)
    d32 = a / np.float32(7.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = w.reshape(n, k // 32, 32) / d32[:, :, None]
        r = np.clip(np.sign(v) * np.floor(np.abs(v.astype(np.float64)) + 0.5), -8, 7)
    r[np.broadcast_to(d32[:, :, None] == 0, r.shape)] = 0
    return r.astype(np.int8).reshape(n, k), d32.astype(np.float16)


def quantize_truncate(w):
    w = np.asarray(w, np.float32)
    n, k = w.shape
    d = q4.block_scales(w)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = w.reshape(n, k // 32, 32) / d.astype(np.float32)[:, :, None]
        r = np.clip(np.trunc(v), -8, 7)
    r[np.broadcast_to(d[:, :, None] == 0, r.shape)] = 0
    return r.astype(np.int8).reshape(n, k), d


@pytest.mark.parametrize("mutant", [quantize_half_even, quantize_div8, quantize_fp32_scale, quantize_truncate])
def test_quantizer_mutants_caught(mutant):
    with pytest.raises(AssertionError):
        pins.pin_scales(mutant, _w())
        pins.pin_codes(mutant, _w())


# ---- packing mutants ------------------------------------------------------

def pack_swapped(q):
    nib = (np.asarray(q).astype(np.int16) & 0xF).astype(np.uint8)
    return (nib[:, 1::2] | (nib[:, 0::2] << 4)).astype(np.uint8)


def unpack_swapped(codes):
    out = q4.unpack(codes)
    out[:, 0::2], out[:, 1::2] = out[:, 1::2].copy(), out[:, 0::2].copy()
    return out


def unpack_unsigned(codes):
    c = np.asarray(codes, np.uint8)
    out = np.empty((c.shape[0], c.shape[1] * 2), np.int8)
    out[:, 0::2] = c & 0xF
    out[:, 1::2] = c >> 4
    return out


def test_swapped_nibbles_caught():
    # a consistent swap in both directions still round-trips; the literal catches it
    pins.pin_roundtrip(pack_swapped, unpack_swapped)
    with pytest.raises(AssertionError):
        pins.pin_pack_literal(pack_swapped)


def test_unsigned_unpack_caught():
    with pytest.raises(AssertionError):
        pins.pin_roundtrip(q4.pack, unpack_unsigned)


# ---- matmul mutants -------------------------------------------------------

def matmul_transposed(x, q, d):
    return np.asarray(x, np.float64) @ q4.dequantize(q, d)


def matmul_drop_last_block(x, q, d):
    qq = np.array(q, copy=True)
    qq[:, -32:] = 0
    return q4.matmul(x, qq, d)


def matmul_scale_shift(x, q, d):
    """Scale of block b applied to block b+1 (an off-by-one block index)."""
    return np.asarray(x, np.float64) @ (q.astype(np.float64) * np.repeat(np.roll(d.astype(np.float64), 1, axis=1), 32, axis=1)).T


def matmul_sign(x, q, d):
    return -q4.matmul(x, q, d)


@pytest.mark.parametrize("mutant", [matmul_transposed, matmul_drop_last_block, matmul_scale_shift, matmul_sign])
def test_matmul_mutants_caught(mutant):
    w = synthetic.weights(64, 64, seed=52)
    x = synthetic.activations(1, 64, seed=53)
    q, d = q4.quantize(w)
    with pytest.raises(AssertionError):
        pins.pin_matmul_exact(mutant, x, q, d)


# ---- A8 mutants -----------------------------------------------------------

def quantize_act_div128(x):
    x32 = np.asarray(x, np.float16).astype(np.float32)
    m, k = x32.shape
    g = x32.reshape(m, k // 64, 64)
    sa = np.max(np.abs(g), axis=2) / np.float32(128.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (g / sa[:, :, None]).astype(np.float64)
    r = np.clip(np.sign(v) * np.floor(np.abs(v) + 0.5), -127, 127)
    r[np.broadcast_to(sa[:, :, None] == 0, r.shape)] = 0
    return r.astype(np.int8).reshape(m, k), sa


def quantize_act_group32(x):
    """Scales per 32 channels instead of 64 (reported at the same shape by taking every other)."""
    x32 = np.asarray(x, np.float16).astype(np.float32)
    m, k = x32.shape
    g = x32.reshape(m, k // 32, 32)
    sa = np.max(np.abs(g), axis=2) / np.float32(127.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (g / sa[:, :, None]).astype(np.float64)
    r = np.clip(np.sign(v) * np.floor(np.abs(v) + 0.5), -127, 127)
    r[np.broadcast_to(sa[:, :, None] == 0, r.shape)] = 0
    return r.astype(np.int8).reshape(m, k), sa[:, 0::2]


def a8_matmul_group_index(qa, sa, q, d):
    """Activation scale indexed by block instead of by 64-channel group."""
    qa64 = qa.astype(np.float64)
    q64 = q.astype(np.float64)
    y = np.zeros((qa.shape[0], q.shape[0]))
    nb = qa.shape[1] // 32
    for b in range(nb):
        sl = slice(32 * b, 32 * b + 32)
        y += (sa.astype(np.float64)[:, min(b, sa.shape[1] - 1)][:, None] * (qa64[:, sl] @ q64[:, sl].T)) * d.astype(np.float64)[:, b][None, :]
    return y


@pytest.mark.parametrize("mutant", [quantize_act_div128, quantize_act_group32])
def test_act_quant_mutants_caught(mutant):
    x = np.concatenate([synthetic.activations(2, 128, seed=54), _special_acts()])
    with pytest.raises(AssertionError):
        pins.pin_act_quant(mutant, x)


def test_a8_group_index_mutant_caught():
    x = synthetic.activations(2, 128, seed=55)
    q, d = q4.quantize(synthetic.weights(3, 128, seed=56))
    qa, sa = a8.quantize_act(x)
    with pytest.raises(AssertionError):
        pins.pin_a8_exact(a8_matmul_group_index, qa, sa, q, d)


# ---- attention-read mutants -------------------------------------------------

def _attn_mutant(scale=None, vis_shift=0, head_of=None, subtract_max=True, swap_kv=False, normalize=True):
    """A copy of the attention oracle with one plausible slip."""
    def fn(q, k_codes, k_scales, v_codes, v_scales, n_kv_heads):
        from oracle import attn
        q64 = np.asarray(q, dtype=np.float16).astype(np.float64)
        m_count, n_q, d = q64.shape
        group = n_q // n_kv_heads
        k = attn.dequantize_cache(k_codes, k_scales, n_kv_heads)
        v = attn.dequantize_cache(v_codes, v_scales, n_kv_heads)
        if swap_kv:
            k, v = v, k
        t = k.shape[0]
        out = np.zeros((m_count, n_q, d))
        for m in range(m_count):
            n_vis = max(1, t - m_count + m + 1 + vis_shift)
            for h in range(n_q):
                g = head_of(h, group, n_kv_heads) if head_of else h // group
                s = k[:n_vis, g, :] @ q64[m, h] * (scale(d) if scale else 1 / np.sqrt(d))
                with np.errstate(over="ignore", invalid="ignore"):
                    p = np.exp(s - np.max(s)) if subtract_max else np.exp(s)
                    if normalize:
                        p = p / np.sum(p)
                out[m, h] = p @ v[:n_vis, g, :]
        return out
    return fn


ATTN_MUTANTS = {
    "scale 1/D": _attn_mutant(scale=lambda d: 1.0 / d),
    "sees one row fewer": _attn_mutant(vis_shift=-1),
    "sees one row more": _attn_mutant(vis_shift=+1),
    "head h % H_kv": _attn_mutant(head_of=lambda h, g, nkv: h % nkv),
    "no max subtracted": _attn_mutant(subtract_max=False),
    "K and V swapped": _attn_mutant(swap_kv=True),
    "weights not normalized": _attn_mutant(normalize=False),
}


@pytest.mark.parametrize("name", list(ATTN_MUTANTS))
def test_attention_mutants_caught(name):
    from test_oracle_attn import ALL_PINS
    fn = ATTN_MUTANTS[name]
    caught = 0
    for pin in ALL_PINS:
        try:
            pin(fn)
        except AssertionError:
            caught += 1
    assert caught > 0, f"no pin catches the mutant '{name}'"
