"""Pins of the oracle's base code, candidate losses, argmin and pack (CPU only).

Against: exact-rational recomputation of every candidate (``exact_ref``), the bounds the
ScaleSweep page proves for MSE (the exhaustive optimum lies in offsets [-3, 7]), and invariants
the method fixes (the base candidate is always scored, so the search never does worse than
max-abs; identity weights = plain MSE; the exhaustive mode equals the widest window).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from exact_ref import E2M1, group_exact

REL = 2e-6   # fp32 loss vs exact: nonnegative terms, each through the rounding of h*d, at most
             # four roundings in its quad's fma chain and two in the final adds: relative error
             # < 8 * 2^-24 ~ 4.8e-7 (the bound is kept at 2e-6)


def _groups(kind: str, n: int, seed: int):
    """Random groups of 16 weights and 16 h values of several shapes."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((n, 16)).astype(np.float32) * 0.02
    h = np.exp(rng.standard_normal((n, 16)) * 2.0).astype(np.float32)
    if kind == "outlier":
        w[np.arange(n), rng.integers(0, 16, n)] *= 30
    elif kind == "student":
        w = (rng.standard_t(4, (n, 16)) * 0.015).astype(np.float32)
    elif kind == "sparse":
        w[rng.random((n, 16)) < 0.7] = 0
    elif kind == "equal":
        w = np.sign(w) * np.float32(0.01) * rng.integers(1, 4, (n, 1)).astype(np.float32)
    elif kind == "hzero":
        h[rng.random((n, 16)) < 0.5] = 0
    elif kind == "hwide":
        h = np.exp(rng.standard_normal((n, 16)) * 6.0).astype(np.float32)
    return w, h


KINDS = ["normal", "outlier", "student", "sparse", "equal", "hzero", "hwide"]
MODES = [("wmse", -9, 6, False), ("mse", -3, 7, False), ("wmse", -8, 7, False),
         ("wmse", 0, 0, True), ("mse", 0, 0, True)]


def _check_group(oracle_mod, w16, h16, S, obj, lo, hi, exh):
    hh = h16 if obj == "wmse" else None
    b, codes, losses = oracle_mod.group_candidates(w16, hh, S, lo, hi, exh)
    ex = group_exact(w16, hh, S, lo, hi, exh)
    assert b == ex["base"]
    if b == 0:
        return None
    assert codes.tolist() == ex["codes"]
    exact = ex["exact_losses"]
    for L32, Le in zip(losses, exact):           # each fp32 loss is the exact one, rounded
        assert abs(Fraction(float(L32)) - Le) <= REL * Le
    r = oracle_mod.scale_search(w16.reshape(1, 16), None if hh is None else hh,
                                oracle_mod.WMSE if obj == "wmse" else oracle_mod.MSE,
                                lo, hi, exh, S)
    c = int(r["scales"][0, 0])
    pos = ex["codes"].index(c)
    best = min(exact)
    assert exact[pos] <= best * (1 + 2 * REL)    # chosen candidate is an exact minimiser
    earlier = exact[:pos]                        # nothing before it is clearly better
    assert all(e >= exact[pos] * (1 - 2 * REL) for e in earlier)
    # the chosen nibbles are the exact-nearest E2M1 codes at that scale, with w's sign
    nib = oracle_mod.unpack_nibbles(r["packed"])[0]
    want = [(8 if np.signbit(w16[j]) else 0) | ex["q_index"][pos][j] for j in range(16)]
    assert nib.tolist() == want
    assert int(r["offset"][0, 0]) == c - b
    return c - b


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("mode", MODES, ids=lambda m: f"{m[0]}{'-exh' if m[3] else m[1:3]}")
def test_against_exact_rational(oracle_mod, kind, mode):
    obj, lo, hi, exh = mode
    n = 12 if exh else 40
    w, h = _groups(kind, n, seed=10 * KINDS.index(kind) + MODES.index(mode))
    S = np.float32(np.abs(w).max() / 2688) if np.abs(w).max() > 0 else np.float32(1)
    for i in range(n):
        _check_group(oracle_mod, w[i], h[i], S, obj, lo, hi, exh)


def test_mse_exhaustive_optimum_inside_scalesweep_window(oracle_mod):
    """ScaleSweep Lemmas 4.1/4.3: the MSE optimum lies in offsets [-3, 7] of the base code.
    Where the fp32 exhaustive argmin lands outside, it may only be by a rounding-level tie."""
    rng = np.random.default_rng(21)
    W = np.concatenate([
        (rng.standard_normal((400, 64)) * 0.02),
        (rng.standard_t(4, (400, 64)) * 0.015),
        (rng.uniform(-1, 1, (400, 64)) * 0.05),
    ]).astype(np.float32)
    S = np.float32(np.abs(W).max() / 1536)
    ex = oracle_mod.scale_search(W, None, oracle_mod.MSE, exhaustive=True, S=S)
    win = oracle_mod.scale_search(W, None, oracle_mod.MSE, -3, 7, False, S)
    off = ex["offset"]
    inside = (off >= -3) & (off <= 7)
    assert inside.mean() > 0.999
    np.testing.assert_array_equal(ex["scales"][inside], win["scales"][inside])
    for r, g in zip(*np.nonzero(~inside)):
        assert win["loss"][r, g] <= ex["loss"][r, g] * (1 + 4 * REL)


def _matrix(seed, out=48, n=128, scale=0.02):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((out, n)) * scale).astype(np.float32)
    W[rng.random(W.shape) < 0.003] *= 25
    h = np.exp(rng.standard_normal(n) * 2).astype(np.float32)
    return W, h, np.float32(np.abs(W).max() / 2688)


def test_search_never_worse_than_base(oracle_mod):
    W, h, S = _matrix(1)
    base = oracle_mod.scale_search(W, h, oracle_mod.WMSE, 0, 0, False, S)
    for lo, hi, exh in ((-9, 6, False), (-8, 7, False), (0, 0, True)):
        r = oracle_mod.scale_search(W, h, oracle_mod.WMSE, lo, hi, exh, S)
        assert (r["loss"] <= base["loss"]).all()


def test_identity_weights_equal_mse(oracle_mod):
    W, h, S = _matrix(2)
    mse = oracle_mod.scale_search(W, None, oracle_mod.MSE, -9, 6, False, S)
    one = oracle_mod.scale_search(W, np.ones_like(h), oracle_mod.WMSE, -9, 6, False, S)
    for k in mse:
        np.testing.assert_array_equal(mse[k], one[k])
    for p in (-6, 4):   # h = 2^p scales every loss exactly by 2^p: same choices
        pw = oracle_mod.scale_search(W, np.full_like(h, 2.0 ** p), oracle_mod.WMSE, -9, 6, False, S)
        np.testing.assert_array_equal(mse["scales"], pw["scales"])
        np.testing.assert_array_equal(mse["loss"] * np.float32(2.0 ** p), pw["loss"])


def test_exhaustive_equals_widest_window(oracle_mod):
    W, h, S = _matrix(3)
    a = oracle_mod.scale_search(W, h, oracle_mod.WMSE, exhaustive=True, S=S)
    b = oracle_mod.scale_search(W, h, oracle_mod.WMSE, -125, 125, False, S)
    for k in ("scales", "packed", "loss", "offset"):
        np.testing.assert_array_equal(a[k], b[k])


def test_window_zero_is_maxabs_rtn_pack(oracle_mod):
    W, h, S = _matrix(4)
    r = oracle_mod.scale_search(W, h, oracle_mod.WMSE, 0, 0, False, S)
    np.testing.assert_array_equal(oracle_mod.pack(W, r["scales"], S), r["packed"])
    assert (r["offset"] == 0).all()
    # base code = E4M3-rounded (amax/6)/S
    amax = np.abs(W).reshape(W.shape[0], -1, 16).max(-1)
    s_star = (amax / np.float32(6)).astype(np.float32) / S
    want = np.maximum(oracle_mod.e4m3_encode(s_star.astype(np.float32)), 1)
    want[amax == 0] = 0
    np.testing.assert_array_equal(r["scales"], want)


def test_zero_groups_and_h_zero_tie_rule(oracle_mod):
    W, h, S = _matrix(5, out=4, n=64)
    W[1, 16:32] = 0
    W[2, 0:16] = -0.0
    r = oracle_mod.scale_search(W, h, oracle_mod.WMSE, -9, 6, False, S)
    assert r["scales"][1, 1] == 0 and r["scales"][2, 0] == 0
    nib = oracle_mod.unpack_nibbles(r["packed"])
    assert (nib[1, 16:32] == 0).all() and (nib[2, 0:16] == 8).all()
    hz = np.zeros_like(h)   # every candidate scores 0: the lowest offset wins
    z = oracle_mod.scale_search(W, hz, oracle_mod.WMSE, -9, 6, False, S)
    nz = z["scales"] > 0
    base = oracle_mod.scale_search(W, hz, oracle_mod.WMSE, 0, 0, False, S)["scales"].astype(int)
    np.testing.assert_array_equal(z["scales"][nz], np.maximum(base[nz] - 9, 1))


def test_clipping_at_top_code(oracle_mod):
    """Groups at the top of the code range: +offsets clip to 126 and are duplicates."""
    W = np.zeros((1, 32), np.float32)
    W[0, :16] = np.linspace(-1, 1, 16)
    W[0, 16:] = np.linspace(-0.3, 0.2, 16)
    S = np.float32(1.0 / 2688)
    r = oracle_mod.scale_search(W, None, oracle_mod.MSE, -3, 7, False, S)
    b, codes, _ = oracle_mod.group_candidates(W[0, :16], None, S, -3, 7, False)
    assert b == 126 and codes.tolist() == [123, 124, 125] + [126] * 8
    assert r["scales"][0, 0] <= 126


def test_row_permutation_and_threads(oracle_mod):
    W, h, S = _matrix(6, out=64)
    perm = np.random.default_rng(0).permutation(64)
    a = oracle_mod.scale_search(W, h, oracle_mod.WMSE, -9, 6, False, S, threads=1)
    b = oracle_mod.scale_search(W[perm], h, oracle_mod.WMSE, -9, 6, False, S, threads=8)
    for k in a:
        np.testing.assert_array_equal(a[k][perm], b[k])


def test_pack_roundtrip_values(oracle_mod):
    """Dequantised codes at the max-abs scales stay within half the widest level gap."""
    W, h, S = _matrix(7, out=8, n=64)
    scales = oracle_mod.scale_search(W, h, oracle_mod.WMSE, 0, 0, False, S)["scales"]
    nib = oracle_mod.unpack_nibbles(oracle_mod.pack(W, scales, S))
    eff, rcp = oracle_mod.scale_tables(S)
    levels = np.array([float(v) for v in E2M1])
    deq = np.where(nib & 8, -1.0, 1.0) * levels[nib & 7] * eff[np.repeat(scales, 16, axis=1)]
    err = np.abs(deq - W)
    step = eff[np.repeat(scales, 16, axis=1)].astype(np.float64)
    assert (err <= 1.0 * step + 1e-12).all()       # at most half the widest level gap (2)
    assert (np.sign(deq[deq != 0]) == np.sign(W[deq != 0])).all()


def test_workload_recipe_shapes():
    from block_scale_search_amd import workloads
    cfg = workloads.CONFIGS["tiny"]
    W = workloads.make_weights(cfg)
    sig = workloads.make_sigma(cfg)
    X, _ = workloads.make_activation_chunk(cfg, sig, 0)
    assert W.shape == (256, 256) and W.dtype == torch.float32
    assert X.shape == (512, 256) and X.dtype == torch.bfloat16
    frac = (W.abs() > 0.2).float().mean().item()
    assert 0.003 < frac < 0.008
