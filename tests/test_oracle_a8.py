"""Pins for the A8 prefill oracle (CPU only)."""

import numpy as np
import pytest

import pins
from oracle import a8, q4
from bit_quantized_weight_amd import synthetic


def _special_acts():
    k = 128
    x = np.zeros((3, k), np.float16)
    # group with absmax 127 -> sa = 1 exactly; ties at +-0.5, +-2.5
    x[0, :6] = [127, -127, 2.5, -2.5, 0.5, -0.5]
    # group 1 of row 0 is all zero -> sa = 0, codes 0
    # a group made of tiny (subnormal fp16) values
    x[1, 0] = np.float16(6e-8)
    x[1, 1] = np.float16(-3e-7)
    x[1, 64:] = np.float16(1.0)
    x[2, :] = synthetic.activations(1, k, seed=40)[0] * np.float16(50)
    return x


def test_hand_group():
    qa, sa = a8.quantize_act(_special_acts())
    assert float(sa[0, 0]) == 1.0
    assert qa[0, :6].tolist() == [127, -127, 3, -3, 1, -1]
    assert float(sa[0, 1]) == 0.0 and not qa[0, 64:].any()
    assert np.all(qa[1, 64:] == 127)


def test_act_quant_exact_rational():
    x = np.concatenate([synthetic.activations(4, 128, seed=41), _special_acts()])
    pins.pin_act_quant(a8.quantize_act, x)


def test_block_sums_exact():
    x = synthetic.activations(3, 128, seed=42)
    q, _ = q4.quantize(synthetic.weights(4, 128, seed=43))
    qa, _ = a8.quantize_act(x)
    pins.pin_block_sums(a8.block_sums, qa, q)


def test_block_sums_extremes():
    """|I| reaches 32 * 127 * 8 = 32512 at the extremes and stays exact."""
    qa = np.full((1, 64), -127, np.int8)
    q = np.full((1, 64), -8, np.int8)
    assert a8.block_sums(qa, q).ravel().tolist() == [32512, 32512]


def test_a8_matmul_exact_rational():
    x = synthetic.activations(2, 128, seed=44)
    q, d = q4.quantize(synthetic.weights(3, 128, seed=45))
    qa, sa = a8.quantize_act(x)
    pins.pin_a8_exact(a8.matmul, qa, sa, q, d)


@pytest.mark.parametrize("k,y16", [(256, 255.875), (5120, 5120.0)])
def test_closed_form_all_ones(k, y16):
    """x = 1, W = 1: sa = fl32(1/127), qa = 127, q = 7, I = 32*127*7 = 28448 per block,
    y = (K/32) * 28448 * sa * d exactly.  Because fl32(1/127) lies just below
    1/127, y falls just below K * (1 - 2**-12); at K = 256 that is just below
    the fp16 tie 255.9375, so the fp16 result is 255.875 (the skinny route,
    exactly on the tie, rounds to 256)."""
    from fractions import Fraction
    q, d = q4.quantize(np.ones((2, k), np.float32))
    qa, sa = a8.quantize_act(np.ones((1, k), np.float16))
    assert np.all(sa == np.float32(1.0) / np.float32(127.0))
    assert Fraction(float(sa[0, 0])) == pins.rne(Fraction(1, 127), pins.F32)
    assert np.all(qa == 127)
    assert np.all(a8.block_sums(qa, q) == 28448)
    y = a8.matmul(qa, sa, q, d)
    exact = (k // 32) * 28448 * Fraction(float(sa[0, 0])) * Fraction(0.142822265625)
    assert exact < k * (1 - Fraction(1, 4096))
    assert np.all(np.abs(y - float(exact)) <= 1e-12 * k)
    assert np.all(y.astype(np.float16) == np.float16(y16))


def test_a8_close_to_w4a16():
    """Information, not parity: the A8 route differs from the fp16-activation
    route only by activation-quantization error (a few percent of RMS)."""
    x = synthetic.activations(16, 1024, seed=46)
    q, d = q4.quantize(synthetic.weights(64, 1024, seed=47))
    ya = a8.prefill(x, q, d)
    yw = q4.matmul(x, q, d)
    rms = np.sqrt(np.mean(yw ** 2))
    assert np.max(np.abs(ya - yw)) < 0.05 * rms
