"""Pins for the oracle's per-token absmax int8 activation quantisation."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from brute import round_half_even

from sparse_linear_layers_amd import synth


def _f(bits):
    return oracle.bf16_bits_to_float(bits)


@pytest.mark.parametrize("T,K", [(8, 64), (32, 256)])
def test_exact_rational_rounding_away_from_ties(T, K):
    x = synth.activations_bf16(f"test/act/{T}x{K}", T, K)
    xq, beta = oracle.act_quant(x)
    xf = _f(x)
    for t in range(T):
        b = Fraction(float(np.abs(xf[t]).max()))
        assert beta[t] == np.float32(float(b))
        for j in range(K):
            q = Fraction(float(xf[t, j])) * 127 / b
            frac = abs(q) - int(abs(q))
            # two float roundings move q by at most ~2^-17 here
            if abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 14):
                assert abs(int(xq[t, j]) - q) <= Fraction(1, 2) + Fraction(1, 1 << 14)
                continue
            assert xq[t, j] == round_half_even(q), (t, j)


def test_argmax_maps_to_127_and_range():
    x = synth.activations_bf16("test/act/argmax", 64, 512)
    xq, beta = oracle.act_quant(x)
    xf = _f(x)
    for t in range(64):
        j = int(np.abs(xf[t]).argmax())
        assert abs(int(xq[t, j])) == 127
        assert np.sign(xq[t, j]) == np.sign(xf[t, j])
    assert np.abs(xq.astype(np.int32)).max() <= 127


def test_zero_token():
    x = np.zeros((3, 64), dtype=np.uint16)
    x[1, 5] = 0x8000  # -0.0
    xq, beta = oracle.act_quant(x)
    assert (xq == 0).all()
    assert (beta == np.float32(1e-5)).all()


@pytest.mark.parametrize("k", [-3, 1, 5])
def test_power_of_two_scaling_is_invisible(k):
    x = synth.activations_bf16("test/act/scale", 16, 128)
    xq, beta = oracle.act_quant(x)
    # multiply the bf16 values by 2^k exactly: adjust the exponent field
    xs = (x.astype(np.int32) + (k << 7)).astype(np.uint16)
    xq2, beta2 = oracle.act_quant(xs)
    assert (xq2 == xq).all()
    assert np.array_equal(beta2, (beta * np.float32(2.0 ** k)).astype(np.float32))


def test_exact_half_ties_round_to_even():
    """With beta = 127 the scale 127/beta is exactly 1, so x~ = Round(x) and
    bf16 half-integers hit the rounding ties exactly (torch.round, the
    guide's module, rounds half to even)."""
    from sparse_linear_layers_amd.synth import float_to_bf16_bits
    vals = np.array([127, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5, 4.5, -126.5, 125.5, 0.25],
                    dtype=np.float32)
    x = float_to_bf16_bits(np.concatenate([vals, np.zeros(4, np.float32)])[None, :])
    assert (oracle.bf16_bits_to_float(x)[0, :12] == vals).all()  # exact in bf16
    xq, beta = oracle.act_quant(x)
    assert beta[0] == 127
    want = [127, 0, 2, 2, 0, -2, -2, 4, 4, -126, 126, 0]
    assert xq[0, :12].tolist() == want
