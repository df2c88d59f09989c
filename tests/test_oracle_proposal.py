"""Pins of the oracle's proposal-centred search (Replay the Curvature §4.1.3-§4.1.4, App. D.2):
a half-window of codes around a per-group proposal plus the incoming scale, which is kept on
ties (CPU only).

Against: exact-rational recomputation of every candidate's loss (``exact_ref``), the reduction
to the plain window search when the proposal is the max-abs base code and there is no incoming
code, the retain-on-tie rule where every loss is equal (h = 0), and the page's guarantee that
keeping the status-quo scale means the local search never increases the loss.
"""
import numpy as np
import pytest

from exact_ref import group_exact, losses_at

REL = 2e-6


def _groups(seed, n=40):
    rng = np.random.default_rng(seed)
    w = (rng.standard_t(4, (n, 16)) * 0.015).astype(np.float32)
    w[rng.random((n, 16)) < 0.05] *= 20
    h = np.exp(rng.standard_normal((n, 16)) * 2.5).astype(np.float32)
    return w, h, rng


@pytest.mark.parametrize("obj", ["wmse", "mse"])
@pytest.mark.parametrize("window", [(-4, 4), (-2, 7), (0, 0)])
def test_proposal_against_exact_rational(oracle_mod, obj, window):
    lo, hi = window
    w, h, rng = _groups(seed=100 + 20 * (lo + 10) + hi + (obj == "mse"))
    S = np.float32(np.abs(w).max() / 2688)
    n = w.shape[0]
    for i in range(n):
        hh = h[i] if obj == "wmse" else None
        base = group_exact(w[i], hh, S, 0, 0)["base"]
        center = int(np.clip(base + rng.integers(-6, 7), 0, 140))     # some outside 1..126
        kind = i % 3
        incoming = 0 if kind == 0 else (center if kind == 1 else int(rng.integers(1, 127)))
        r = oracle_mod.scale_search_proposal(
            w[i].reshape(1, 16), hh, oracle_mod.WMSE if obj == "wmse" else oracle_mod.MSE, lo, hi,
            np.array([[center]], np.uint8), np.array([[incoming]], np.uint8), S)
        c = int(r["scales"][0, 0])
        cen = min(max(center, 1), 126)
        window_codes = [min(max(cen + o, 1), 126) for o in range(lo, hi + 1)]
        cands = ([incoming] if 1 <= incoming <= 126 else []) + window_codes
        exact, qidx = losses_at(w[i], hh, S, cands)
        assert c in cands
        pos = cands.index(c)
        best = min(exact)
        assert exact[pos] <= best * (1 + 2 * REL)                   # an exact minimiser
        assert all(e >= exact[pos] * (1 - 2 * REL) for e in exact[:pos])  # none earlier clearly better
        if 1 <= incoming <= 126:
            # the incoming scale is kept unless a candidate is clearly better
            assert exact[pos] <= exact[0] * (1 + 2 * REL)
            if all(exact[0] < e * (1 - 2 * REL) for e in exact[1:]) and c != incoming:
                raise AssertionError("incoming scale dropped for a worse candidate")
        nib = oracle_mod.unpack_nibbles(r["packed"])[0]
        want = [(8 if np.signbit(w[i][j]) else 0) | qidx[pos][j] for j in range(16)]
        assert nib.tolist() == want
        assert int(r["offset"][0, 0]) == c - cen


def _matrix(seed, out=40, n=256):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((out, n)) * 0.02).astype(np.float32)
    W[rng.random(W.shape) < 0.004] *= 25
    W[3, 16:48] = 0.0                                                 # two zero groups
    h = np.exp(rng.standard_normal(n) * 2).astype(np.float32)
    return W, h, np.float32(np.abs(W).max() / 2688), rng


@pytest.mark.parametrize("obj,lo,hi", [("wmse", -4, 4), ("mse", -3, 7), ("wmse", -9, 6)])
def test_proposal_at_base_without_incoming_is_the_window_search(oracle_mod, obj, lo, hi):
    W, h, S, _ = _matrix(31)
    O = oracle_mod.WMSE if obj == "wmse" else oracle_mod.MSE
    hh = h if obj == "wmse" else None
    base = oracle_mod.scale_search(W, None, oracle_mod.MSE, 0, 0, False, S)["scales"]
    p = oracle_mod.scale_search_proposal(W, hh, O, lo, hi, base, None, S)
    q = oracle_mod.scale_search(W, hh, O, lo, hi, False, S)
    for k in ("scales", "packed", "loss", "offset"):
        np.testing.assert_array_equal(p[k], q[k], err_msg=k)


def test_proposal_with_the_window_argmin_as_incoming_keeps_it(oracle_mod):
    W, h, S, _ = _matrix(32)
    base = oracle_mod.scale_search(W, None, oracle_mod.MSE, 0, 0, False, S)["scales"]
    q = oracle_mod.scale_search(W, h, oracle_mod.WMSE, -4, 4, False, S)
    p = oracle_mod.scale_search_proposal(W, h, oracle_mod.WMSE, -4, 4, base, q["scales"], S)
    np.testing.assert_array_equal(p["scales"], q["scales"])
    np.testing.assert_array_equal(p["loss"], q["loss"])
    np.testing.assert_array_equal(p["packed"], q["packed"])


def test_proposal_retains_incoming_on_ties(oracle_mod):
    """h = 0 makes every candidate's loss 0: the incoming code is kept; without one, the
    window's lowest code wins."""
    W, h, S, rng = _matrix(33)
    gpr = W.shape[1] // 16
    center = rng.integers(20, 110, (W.shape[0], gpr)).astype(np.uint8)
    incoming = rng.integers(1, 127, (W.shape[0], gpr)).astype(np.uint8)
    z = np.zeros_like(h)
    p = oracle_mod.scale_search_proposal(W, z, oracle_mod.WMSE, -4, 4, center, incoming, S)
    nz = np.abs(W).reshape(W.shape[0], gpr, 16).max(-1) > 0
    np.testing.assert_array_equal(p["scales"][nz], incoming[nz])
    assert (p["scales"][~nz] == 0).all()
    p2 = oracle_mod.scale_search_proposal(W, z, oracle_mod.WMSE, -4, 4, center, None, S)
    np.testing.assert_array_equal(p2["scales"][nz], np.clip(center.astype(int) - 4, 1, 126)[nz])


def test_proposal_never_increases_the_incoming_loss(oracle_mod):
    """Keeping the status-quo scale guarantees the local search does not increase the loss."""
    W, h, S, rng = _matrix(34)
    gpr = W.shape[1] // 16
    base = oracle_mod.scale_search(W, None, oracle_mod.MSE, 0, 0, False, S)["scales"].astype(int)
    center = np.clip(base + rng.integers(-5, 6, base.shape), 1, 126).astype(np.uint8)
    incoming = np.clip(base + rng.integers(-12, 13, base.shape), 1, 126).astype(np.uint8)
    p = oracle_mod.scale_search_proposal(W, h, oracle_mod.WMSE, -4, 4, center, incoming, S)
    # loss at the incoming code alone: a one-code window centred on it
    at_inc = oracle_mod.scale_search_proposal(W, h, oracle_mod.WMSE, 0, 0, incoming, None, S)
    assert (p["loss"] <= at_inc["loss"]).all()
    nz = np.abs(W).reshape(W.shape[0], gpr, 16).max(-1) > 0      # zero groups get scale 0
    moved = (p["scales"] != incoming) & nz
    assert (p["loss"][moved] < at_inc["loss"][moved]).all()


def test_proposal_center_clamped(oracle_mod):
    W, h, S, _ = _matrix(35, out=8)
    gpr = W.shape[1] // 16
    lo_c = np.zeros((8, gpr), np.uint8)
    hi_c = np.full((8, gpr), 200, np.uint8)
    a = oracle_mod.scale_search_proposal(W, h, oracle_mod.WMSE, -4, 4, lo_c, None, S)
    b = oracle_mod.scale_search_proposal(W, h, oracle_mod.WMSE, -4, 4, np.ones_like(lo_c), None, S)
    np.testing.assert_array_equal(a["scales"], b["scales"])
    np.testing.assert_array_equal(a["offset"], b["offset"])
    c = oracle_mod.scale_search_proposal(W, h, oracle_mod.WMSE, -4, 4, hi_c, None, S)
    d = oracle_mod.scale_search_proposal(W, h, oracle_mod.WMSE, -4, 4, np.full_like(hi_c, 126), None, S)
    np.testing.assert_array_equal(c["scales"], d["scales"])
