"""Pins for the oracle's per-row absmean scale and ternary codes (CPU only)."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from brute import exact_mean_abs, exact_to_bf16, exact_to_f32, f32, round_half_even, unpack_bits

from sparse_linear_layers_amd import synth


def _bf16_bits_of(f):
    return int(np.array([f], dtype=np.float32).view(np.uint32)[0] >> 16)


@pytest.mark.parametrize("cols", [8, 64, 256])
def test_row_scale_is_exact_rational_mean(cols):
    W = synth.latent_weight(f"test/scale/{cols}", 24, cols)
    g, gb = oracle.row_scale(W)
    for r in range(W.shape[0]):
        q = exact_mean_abs(W[r])
        assert g[r] == np.float32(max(exact_to_f32(q), f32(1e-5))), r
        # bf16 copy is the nearest-even bf16 of the float scale
        assert gb[r] == _bf16_bits_of(exact_to_bf16(Fraction(float(g[r])))), r


def test_row_scale_masked_variant_sums_kept_weights_only():
    W = synth.latent_weight("test/scale/masked", 12, 64)
    mb = oracle.nm_mask(W, 3, 4)
    M = unpack_bits(mb, 12, 64)
    g, _ = oracle.row_scale(W, mb, from_masked=True)
    for r in range(12):
        q = sum((Fraction(abs(float(v))) for v in W[r][M[r]]), Fraction(0)) / 64
        assert g[r] == np.float32(exact_to_f32(q))
    g_dense, _ = oracle.row_scale(W)
    assert (g < g_dense).all()  # dropping the smallest quarter lowers the mean


def test_zero_row_clamps_to_epsilon_and_codes_vanish():
    W = np.zeros((2, 16), dtype=np.float32)
    W[1, 3] = 1e-9  # mean far below the clamp
    g, _ = oracle.row_scale(W)
    assert (g == np.float32(1e-5)).all()
    codes = oracle.ternary_codes(W, None, g)
    assert (codes == 0).all()


def _boundary_dense(gamma: np.ndarray, cols: int, seed: int) -> np.ndarray:
    """Weights concentrated at and one ulp around gamma/2 and 3*gamma/2."""
    r = np.random.default_rng(seed)
    rows = gamma.shape[0]
    W = np.empty((rows, cols), dtype=np.float32)
    for i in range(rows):
        h = np.float32(gamma[i] / np.float32(2))
        t = np.float32(gamma[i] * np.float32(1.5))
        cands = [h, np.nextafter(h, np.float32(0)), np.nextafter(h, np.float32(1)),
                 t, np.nextafter(t, np.float32(0)), np.nextafter(t, np.float32(10)),
                 np.float32(0), gamma[i], np.float32(gamma[i] * 4)]
        v = r.choice(np.array(cands, dtype=np.float32), size=cols)
        s = r.choice(np.array([-1, 1], dtype=np.float32), size=cols)
        W[i] = (v * s).astype(np.float32)
    return W


def test_codes_match_closed_form_on_boundary_dense_inputs():
    r = np.random.default_rng(7)
    gamma = (r.uniform(1e-5, 1.0, size=64)).astype(np.float32)
    gamma[:4] = [1e-5, 0.02, 0.5, 1.0]
    W = _boundary_dense(gamma, 256, 8)
    codes = oracle.ternary_codes(W, None, gamma)
    half = (gamma / np.float32(2))[:, None]
    closed = (np.sign(W) * (np.abs(W) > half)).astype(np.int8)
    assert (codes == closed).all()
    assert set(np.unique(codes)) <= {-1, 0, 1}


def test_codes_match_exact_rounding_of_the_quotient():
    W = synth.latent_weight("test/codes/exact", 16, 64)
    gamma, _ = oracle.row_scale(W)
    codes = oracle.ternary_codes(W, None, gamma)
    for i in range(16):
        for j in range(64):
            q = Fraction(float(W[i, j])) / Fraction(float(gamma[i]))
            frac = abs(q) - int(abs(q))
            if abs(frac - Fraction(1, 2)) < Fraction(1, 1 << 20):
                continue  # within float rounding of a tie: decided in float
            e = max(-1, min(1, round_half_even(q)))
            assert codes[i, j] == e, (i, j)


def test_masked_positions_are_zero():
    W = synth.latent_weight("test/codes/mask", 32, 128)
    mb = oracle.nm_mask(W, 2, 4)
    g, _ = oracle.row_scale(W)
    codes = oracle.ternary_codes(W, mb, g)
    M = unpack_bits(mb, 32, 128)
    assert (codes[~M] == 0).all()
    dense = oracle.ternary_codes(W, None, g)
    assert (codes[M] == dense[M]).all()
    # quantise-then-mask equals mask-then-quantise for a fixed gamma
    Wm = np.where(M, W, np.float32(0)).astype(np.float32)
    assert (oracle.ternary_codes(Wm, None, g) == codes).all()


def test_zero_fraction_statistics():
    """For N(0, 0.02) weights the dense ternary zero fraction is about
    P(|z| <= 0.5 E|z|) = 0.31, inside the guide's "30% to 40%" remark
    ("Natural Affinity" section); 3:4 masking leaves about 63% of weights nonzero."""
    W = synth.latent_weight("test/codes/stats", 256, 1024)
    g, _ = oracle.row_scale(W)
    dense = oracle.ternary_codes(W, None, g)
    z = float((dense == 0).mean())
    assert 0.30 < z < 0.32
    sparse = oracle.ternary_codes(W, oracle.nm_mask(W, 3, 4), g)
    # dropping the smallest of four removes a nonzero code only when the
    # group had no zero: nonzero density falls from 0.69 to about 0.63
    assert 0.62 < float((sparse != 0).mean()) < 0.65


def test_bf16_rounding_ties_and_neighbours():
    """bf16 rounding of exact ties and one ulp either side against exact
    rational nearest-even rounding."""
    pats = []
    for hi in (0x3F80, 0x3F81, 0x3C23, 0x3C24, 0x0080, 0x4780):
        for lo in (0x7FFF, 0x8000, 0x8001, 0x0000, 0xFFFF):
            pats.append((hi << 16) | lo)
    fs = np.array(pats, dtype=np.uint32).view(np.float32)
    for f in fs:
        got = oracle.bf16_rne(float(f))
        assert got == _bf16_bits_of(exact_to_bf16(Fraction(float(f)))), hex(int(np.float32(f).view(np.uint32)))
