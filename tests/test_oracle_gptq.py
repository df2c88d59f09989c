"""Pins of the oracle's GPTQ with the window search as local quantiser (H-Scale App. B;
Replay the Curvature §3: columns in sequence, one shared Hessian factor, rows independent).

Against: the identity factor (no propagation: exactly the window search), an independent
binary64 textbook GPTQ written here (given the oracle's group scales: codes agree except at
rounding ties, trajectories agree to binary32 accuracy), and GPTQ's purpose: a lower
layer-output error than rounding each group with the same search.
"""
import numpy as np
import pytest

from exact_ref import E2M1, E4M3


def _layer(seed, out=32, n=128, T=512):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((out, n)) * 0.02).astype(np.float32)
    W[rng.random(W.shape) < 0.01] *= 15
    # correlated activations so that the Hessian is far from diagonal
    A = rng.standard_normal((n, n)) * 0.3 + np.eye(n)
    X = (rng.standard_normal((T, n)) @ A * np.exp(rng.standard_normal(n) * 0.7)).astype(np.float32)
    return W, X


def _factor(X, damp=0.01):
    """U: upper factor of the damped inverse Hessian, (H + damp mean(diag) I)^-1 = U^T U."""
    H = X.astype(np.float64).T @ X.astype(np.float64)
    H += damp * np.mean(np.diag(H)) * np.eye(H.shape[0])
    Hinv = np.linalg.inv(H)
    L = np.linalg.cholesky(Hinv)                # Hinv = L L^T, so U = L^T
    return L.T.astype(np.float32), np.diag(H).astype(np.float32)


def test_identity_factor_is_the_window_search(oracle_mod):
    W, _ = _layer(1)
    h = np.exp(np.random.default_rng(2).standard_normal(128)).astype(np.float32)
    S = np.float32(np.abs(W).max() / 2688)
    U = np.eye(128, dtype=np.float32)
    g = oracle_mod.gptq(W, U, h, oracle_mod.WMSE, -9, 6, S)
    q = oracle_mod.scale_search(W, h, oracle_mod.WMSE, -9, 6, False, S)
    np.testing.assert_array_equal(g["scales"], q["scales"])
    np.testing.assert_array_equal(g["packed"], q["packed"])
    np.testing.assert_array_equal(g["W_final"], W)


def _textbook_gptq(W, U, scales, S):
    """Binary64 GPTQ at given group scales: per column, round to the nearest E2M1 level at the
    group's effective scale, error / U[j,j], subtract error * U[j, k] from every later column."""
    lv = np.array([float(v) for v in E2M1])
    dec = np.array([float(v) for v in E4M3])
    out, n = W.shape
    w = W.astype(np.float64).copy()
    codes = np.zeros((out, n), dtype=np.int64)
    near = np.zeros((out, n), dtype=bool)
    mids = (lv[1:] + lv[:-1]) / 2
    for j in range(n):
        c = scales[:, j // 16].astype(np.int64)
        eff = np.float64(S) * dec[c]
        x = np.where(c > 0, np.abs(w[:, j]) / np.where(eff > 0, eff, 1), 0.0)
        idx = np.searchsorted(mids, x)                    # nearest level (ties: either side)
        near[:, j] = np.min(np.abs(x[:, None] - mids[None, :]), axis=1) < 1e-4 * np.maximum(x, 1e-3)
        codes[:, j] = idx | np.where(np.signbit(w[:, j]), 8, 0)
        v = np.sign(w[:, j]) * lv[idx] * eff
        err = (w[:, j] - v) / U[j, j]
        w[:, j + 1:] -= err[:, None] * U[j, j + 1:].astype(np.float64)[None, :]
    return codes, w, near


def test_against_textbook_binary64_gptq(oracle_mod):
    W, X = _layer(3)
    U, h = _factor(X)
    S = np.float32(np.abs(W).max() / 2688)
    g = oracle_mod.gptq(W, U, h, oracle_mod.WMSE, -9, 6, S)
    codes, w64, near = _textbook_gptq(W, U, g["scales"], S)
    nib = oracle_mod.unpack_nibbles(g["packed"]).astype(np.int64)
    diff = nib != codes
    # binary32 against binary64: codes may only differ where the value sits at a rounding tie,
    # or downstream of such a difference in the same row
    first = np.argmax(diff, axis=1)
    rows = np.nonzero(diff.any(axis=1))[0]
    assert diff.mean() < 0.02
    for r in rows:
        assert near[r, first[r]], f"row {r}: first code difference at column {first[r]} is not a tie"
    ok = ~diff.any(axis=1)
    assert ok.mean() > 0.8
    np.testing.assert_allclose(g["W_final"][ok], w64[ok], rtol=2e-3, atol=2e-5)


def test_gptq_lowers_the_output_error(oracle_mod):
    W, X = _layer(4, out=48, n=128, T=1024)
    U, h = _factor(X)
    S = np.float32(np.abs(W).max() / 2688)
    g = oracle_mod.gptq(W, U, h, oracle_mod.WMSE, -9, 6, S)
    q = oracle_mod.scale_search(W, h, oracle_mod.WMSE, -9, 6, False, S)
    e_gptq = oracle_mod.output_error(X, W, g["packed"], g["scales"], S).sum()
    e_rtn = oracle_mod.output_error(X, W, q["packed"], q["scales"], S).sum()
    assert e_gptq < 0.8 * e_rtn


def test_rows_are_independent(oracle_mod):
    W, X = _layer(5, out=16, n=64, T=256)
    U, h = _factor(X)
    S = np.float32(np.abs(W).max() / 2688)
    g = oracle_mod.gptq(W, U, h, oracle_mod.WMSE, -8, 7, S)
    perm = np.random.default_rng(6).permutation(16)
    p = oracle_mod.gptq(W[perm], U, h, oracle_mod.WMSE, -8, 7, S, threads=1)
    np.testing.assert_array_equal(p["scales"], g["scales"][perm])
    np.testing.assert_array_equal(p["packed"], g["packed"][perm])
