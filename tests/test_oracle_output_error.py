"""Pins of the oracle's dequantisation and layer-output error (CPU only).

The output error err[o] = sum_t (sum_i x_ti (w_oi - w_hat_oi))^2 is H-Scale's layer-output
reconstruction criterion (§3), the quantity its activation-loss comparison of Min-Max,
MSE-guided and Hessian-guided scales reports. Against: a second dequantisation built from the
E2M1/E4M3 bit layouts (``exact_ref``), closed forms (zero error for already-quantised weights,
the squared residual norm for identity activations, exact scaling by 4 when X doubles), brute
force in exact rationals on a tiny layer, and the pages' claim that Hessian-guided scales lower
the output error relative to max-abs scales.
"""
from fractions import Fraction

import numpy as np

from exact_ref import E2M1, E4M3


def _layer(seed, out=24, n=128, T=96):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((out, n)) * 0.02).astype(np.float32)
    W[rng.random(W.shape) < 0.01] *= 20
    W[2, :16] = 0.0                                            # a zero group
    sigma = np.exp(rng.standard_normal(n) * 1.0)
    X = (rng.standard_normal((T, n)) * sigma).astype(np.float32)
    return W, X, np.float32(np.abs(W).max() / 2688)


def _dequant_from_bit_layouts(packed, scales, S):
    out, half = packed.shape
    n = 2 * half
    lv = np.array([float(v) for v in E2M1], dtype=np.float32)
    dec = np.array([float(v) for v in E4M3], dtype=np.float32)
    nib = np.stack([packed & 15, packed >> 4], axis=-1).reshape(out, n)
    c = np.repeat(scales, 16, axis=1)
    eff = (np.float32(S) * dec[c]).astype(np.float32)            # one binary32 product
    mag = (lv[nib & 7] * eff).astype(np.float32)                  # one binary32 product
    mag[c == 0] = 0.0
    return np.where(nib & 8, -mag, mag).astype(np.float32)


def test_dequant_matches_bit_layout_formulation(oracle_mod):
    W, X, S = _layer(1)
    for lo, hi in ((0, 0), (-9, 6)):
        r = oracle_mod.scale_search(W, None, oracle_mod.MSE, lo, hi, False, S)
        a = oracle_mod.dequant(r["packed"], r["scales"], S)
        b = _dequant_from_bit_layouts(r["packed"], r["scales"], S)
        np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))
    # random codes over the whole nibble and scale range, zero scale bytes included
    rng = np.random.default_rng(2)
    packed = rng.integers(0, 256, (7, 32), dtype=np.uint8)
    scales = rng.integers(0, 127, (7, 4), dtype=np.uint8)
    scales[0, 0] = 0
    a = oracle_mod.dequant(packed, scales, S)
    b = _dequant_from_bit_layouts(packed, scales, S)
    np.testing.assert_array_equal(a.view(np.uint32), b.view(np.uint32))


def test_output_error_zero_for_quantised_weights(oracle_mod):
    W, X, S = _layer(3)
    r = oracle_mod.scale_search(W, None, oracle_mod.MSE, -3, 7, False, S)
    W_hat = oracle_mod.dequant(r["packed"], r["scales"], S)
    # re-quantising the dequantised weights at the same scales reproduces the codes, and the
    # output error of W_hat against its own codes is exactly 0
    assert (oracle_mod.output_error(X, W_hat, r["packed"], r["scales"], S) == 0).all()


def test_output_error_identity_activations_is_residual_norm(oracle_mod):
    W, _, S = _layer(4, n=64)
    r = oracle_mod.scale_search(W, None, oracle_mod.MSE, 0, 0, False, S)
    X = np.eye(64, dtype=np.float32)
    err = oracle_mod.output_error(X, W, r["packed"], r["scales"], S)
    e = W.astype(np.float64) - oracle_mod.dequant(r["packed"], r["scales"], S).astype(np.float64)
    np.testing.assert_allclose(err, (e * e).sum(axis=1), rtol=1e-14, atol=0)


def test_output_error_scales_by_four(oracle_mod):
    W, X, S = _layer(5)
    r = oracle_mod.scale_search(W, None, oracle_mod.MSE, 0, 0, False, S)
    a = oracle_mod.output_error(X, W, r["packed"], r["scales"], S)
    b = oracle_mod.output_error(2 * X, W, r["packed"], r["scales"], S)
    np.testing.assert_array_equal(b, 4 * a)


def test_output_error_brute_force_exact(oracle_mod):
    W, X, S = _layer(6, out=3, n=32, T=5)
    r = oracle_mod.scale_search(W, None, oracle_mod.MSE, -2, 2, False, S)
    W_hat = _dequant_from_bit_layouts(r["packed"], r["scales"], S)
    err = oracle_mod.output_error(X, W, r["packed"], r["scales"], S)
    for o in range(3):
        tot = Fraction(0)
        for t in range(5):
            y = sum(Fraction(float(X[t, i])) * (Fraction(float(W[o, i])) - Fraction(float(W_hat[o, i])))
                    for i in range(32))
            tot += y * y
        assert abs(Fraction(float(err[o])) - tot) <= tot * Fraction(1, 10 ** 12)


def test_hessian_guided_scales_lower_the_output_error(oracle_mod):
    """H-Scale §3 and ScaleSweep's evaluation: Hessian-weighted scales reduce the layer-output
    error relative to max-abs scales (on independent-channel activations the diagonal Hessian
    is the whole Hessian up to sampling noise)."""
    W, X, S = _layer(7, out=48, n=256, T=512)
    _, h = oracle_mod.diag_hessian(X)
    base = oracle_mod.scale_search(W, None, oracle_mod.MSE, 0, 0, False, S)
    wmse = oracle_mod.scale_search(W, h, oracle_mod.WMSE, -9, 6, False, S)
    e_base = oracle_mod.output_error(X, W, base["packed"], base["scales"], S).sum()
    e_wmse = oracle_mod.output_error(X, W, wmse["packed"], wmse["scales"], S).sum()
    assert e_wmse < 0.9 * e_base
