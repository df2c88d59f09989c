"""Property tests of the oracle's search (CPU, hypothesis): random and adversarial groups of 16.

Strategies draw groups with all-zero and single-element patterns, repeated magnitudes, values
placed on E2M1 rounding midpoints of some candidate scale, magnitudes from 2^-30 to 2^20 (base
codes that underflow to code 1 and that saturate at 126), and h with zeros and a range of 2^±60.
Checked against the method's own guarantees, not the oracle's formula: the chosen loss never
exceeds the base (max-abs) candidate's ([SR] §4.1.4: keeping the incoming scale); identity h
gives exactly MSE ([HS] §3: the diagonal weighting reduces to MSE); the window [0, 0] is max-abs
RTN; the exhaustive mode equals the widest window; the chosen code is an exact minimiser of the
rational loss (within the binary32 rounding bound) with no clearly better earlier candidate.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from exact_ref import group_exact

REL = 2e-6
MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)


@st.composite
def groups(draw):
    kind = draw(st.sampled_from(["normal", "zero", "single", "repeat", "midpoint", "wide"]))
    e = draw(st.integers(-30, 20))
    seed = draw(st.integers(0, 2 ** 32 - 1))
    rng = np.random.default_rng(seed)
    if kind == "zero":
        w = np.zeros(16)
        if draw(st.booleans()):
            w[rng.random(16) < 0.5] = -0.0
    elif kind == "single":
        w = np.zeros(16)
        w[rng.integers(0, 16)] = rng.standard_normal() * 2.0 ** e
    elif kind == "repeat":
        w = np.sign(rng.standard_normal(16)) * 2.0 ** e * rng.integers(1, 4)
    elif kind == "midpoint":
        # magnitudes on E2M1 midpoints of one candidate scale 2^e (times the global scale below)
        w = np.array([rng.choice(MIDPOINTS) for _ in range(16)]) * 2.0 ** e
        w *= np.sign(rng.standard_normal(16))
    elif kind == "wide":
        w = rng.standard_normal(16) * 2.0 ** rng.integers(-20, 20, 16).astype(float) * 2.0 ** (e // 4)
    else:
        w = rng.standard_normal(16) * 2.0 ** e
    h = np.exp(rng.standard_normal(16) * draw(st.floats(0.0, 6.0)))
    if draw(st.booleans()):
        h[rng.random(16) < 0.3] = 0.0
    if draw(st.booleans()):
        h *= 2.0 ** draw(st.integers(-60, 60))
    # a global scale that puts this group anywhere from deep underflow to saturation
    S = np.float32(2.0 ** draw(st.integers(-40, 10)))
    return w.astype(np.float32), h.astype(np.float32), S


SETTINGS = settings(max_examples=150, deadline=None,
                    suppress_health_check=[HealthCheck.function_scoped_fixture])


@SETTINGS
@given(g=groups(), obj=st.sampled_from(["mse", "wmse"]),
       window=st.sampled_from([(-9, 6), (-3, 7), (-8, 7), (-2, 2), (0, 5)]))
def test_chosen_is_exact_minimiser_and_never_worse_than_base(oracle_mod, g, obj, window):
    w, h, S = g
    hh = h if obj == "wmse" else None
    lo, hi = window
    r = oracle_mod.scale_search(w.reshape(1, 16), hh, oracle_mod.WMSE if obj == "wmse" else oracle_mod.MSE,
                                lo, hi, False, float(S))
    base = oracle_mod.scale_search(w.reshape(1, 16), hh,
                                   oracle_mod.WMSE if obj == "wmse" else oracle_mod.MSE, 0, 0, False,
                                   float(S))
    assert r["loss"][0, 0] <= base["loss"][0, 0]
    if not np.any(w):
        assert r["scales"][0, 0] == 0 and r["loss"][0, 0] == 0
        return
    ex = group_exact(w, hh, S, lo, hi, False)
    c = int(r["scales"][0, 0])
    pos = ex["codes"].index(c)
    exact = ex["exact_losses"]
    assert exact[pos] <= min(exact) * (1 + 2 * REL)
    assert all(e >= exact[pos] * (1 - 2 * REL) for e in exact[:pos])


@SETTINGS
@given(g=groups())
def test_identity_h_is_mse_and_exhaustive_is_widest_window(oracle_mod, g):
    w, _, S = g
    W = w.reshape(1, 16)
    mse = oracle_mod.scale_search(W, None, oracle_mod.MSE, -9, 6, False, float(S))
    one = oracle_mod.scale_search(W, np.ones(16, np.float32), oracle_mod.WMSE, -9, 6, False, float(S))
    for k in mse:
        np.testing.assert_array_equal(mse[k], one[k])
    h = np.abs(w) + np.float32(1.0)
    a = oracle_mod.scale_search(W, h, oracle_mod.WMSE, exhaustive=True, S=float(S))
    b = oracle_mod.scale_search(W, h, oracle_mod.WMSE, -125, 125, False, float(S))
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])
    z = oracle_mod.scale_search(W, h, oracle_mod.WMSE, 0, 0, False, float(S))
    np.testing.assert_array_equal(oracle_mod.pack(W, z["scales"], float(S)), z["packed"])
