"""Pins of the oracle's element formats (CPU only).

E2M1: the levels against the bit layout and the golden file; the tie table; a second,
independent nearest-value formulation over dense sets of binary32 inputs.
E4M3: decode and encode against torch's float8_e4m3fn (a library routine), the code-space
facts the ScaleSweep page states (126 positive finite values; offsets -3, -8 and +7 against the
ratios 4/5, 1/2 and 12/7).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from exact_ref import E2M1, E4M3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_levels():
    with open(os.path.join(GOLDEN, "e2m1_levels.txt")) as f:
        rows = [l for l in f if l.strip() and not l.startswith("#")]
    return [float(v) for v in rows[0].split()]


def _constants():
    with open(os.path.join(GOLDEN, "pages_constants.json")) as f:
        return json.load(f)


def test_e2m1_levels_match_bit_layout_and_golden(oracle_mod):
    golden = _golden_levels()
    assert golden == [float(v) for v in E2M1]
    assert [oracle_mod.e2m1_level(i) for i in range(8)] == golden
    # the H-Scale microcase code pattern consists of signed E2M1 levels
    for v in _constants()["microcase_fp4_pattern"]["value"]:
        assert abs(v) in golden


def test_e2m1_tie_table_and_saturation(oracle_mod):
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 6.5, 12.0, 1e30, 0.0],
                 dtype=np.float32)
    want = [0, 2, 2, 4, 4, 6, 6, 7, 7, 7, 7, 0]  # ties to the even index, >6 saturates
    assert oracle_mod.e2m1_index(x).tolist() == want
    up = np.nextafter(x[:7], np.float32(np.inf))
    dn = np.nextafter(x[:7], np.float32(0))
    assert oracle_mod.e2m1_index(up).tolist() == [1, 2, 3, 4, 5, 6, 7]
    assert oracle_mod.e2m1_index(dn).tolist() == [0, 1, 2, 3, 4, 5, 6]


def _nearest_even_f64(x32: np.ndarray, levels) -> np.ndarray:
    """Second formulation: argmin |x - v| in float64 (exact for these inputs), ties -> even."""
    x = x32.astype(np.float64)
    lv = np.asarray(levels, dtype=np.float64)
    dist = np.abs(x[:, None] - lv[None, :])
    best = dist.min(axis=1, keepdims=True)
    score = (dist == best) * np.where(np.arange(len(lv)) % 2 == 0, 2, 1)[None, :]
    return score.argmax(axis=1).astype(np.uint8)


def _dense_around(points, span_ulps: int):
    out = []
    for p in points:
        bits = np.float32(p).view(np.uint32).astype(np.int64)
        rng = np.arange(max(0, bits - span_ulps), bits + span_ulps + 1, dtype=np.int64)
        out.append(rng.astype(np.uint32).view(np.float32))
    return np.concatenate(out)


def test_e2m1_dense_vs_second_formulation(oracle_mod):
    levels = [float(v) for v in E2M1]
    mids = [(levels[i] + levels[i + 1]) / 2 for i in range(7)]
    rng = np.random.default_rng(7)
    xs = np.concatenate([
        _dense_around(mids + levels[1:], 1 << 14),
        rng.uniform(0, 16, 1 << 21).astype(np.float32),
        (rng.integers(0, 0x41800000, 1 << 20, dtype=np.int64).astype(np.uint32)).view(np.float32),
        np.array([0.0, np.finfo(np.float32).tiny, 1e-45, 3e38], dtype=np.float32),
    ])
    # float64 distances are exact for 2^-20 <= x < 2^20; below, 0 is plainly nearest; above,
    # 6 is.
    mid = (xs >= 2.0 ** -20) & (xs < 2.0 ** 20)
    got = oracle_mod.e2m1_index(xs)
    want = _nearest_even_f64(xs, levels)
    np.testing.assert_array_equal(got[mid], want[mid])
    assert (got[xs < 2.0 ** -20] == 0).all() and (got[xs >= 2.0 ** 20] == 7).all()


def test_e4m3_decode_vs_torch(oracle_mod):
    torch_vals = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    ours = np.array([oracle_mod.e4m3_value(c) for c in range(127)])
    np.testing.assert_array_equal(ours, torch_vals)
    np.testing.assert_array_equal(ours, np.array([float(v) for v in E4M3]))
    # 0x7F is not a finite value in this variant
    assert torch.isnan(torch.tensor([127], dtype=torch.uint8).view(torch.float8_e4m3fn).float())


def test_e4m3_code_space_facts(oracle_mod):
    c = _constants()
    vals = [oracle_mod.e4m3_value(k) for k in range(127)]
    positive = [v for v in vals if v > 0]
    assert len(positive) == c["e4m3_positive_finite_count"]["value"]
    assert all(vals[k] < vals[k + 1] for k in range(126))
    assert vals[126] == 448.0 and vals[1] == 2.0 ** -9
    for k in range(8, 119):          # octave relation of normal codes: -8 is exactly one half
        assert vals[k + 8] == 2 * vals[k]
    # ScaleSweep bounds in bit-pattern space (ratios to the base code's value, normal range)
    ratios = {o: [Fraction(vals[b + o]) / Fraction(vals[b]) for b in range(16, 119)]
              for o in (-8, -4, -3, 6, 7)}
    assert all(r == Fraction(1, 2) for r in ratios[-8])
    assert max(ratios[-4]) < Fraction(4, 5)          # -4 is already below 4/5
    assert max(ratios[-3]) >= Fraction(4, 5)         # ... while -3 can still reach it
    assert min(ratios[7]) > Fraction(12, 7)          # +7 always clears 12/7
    assert max(ratios[6]) >= Fraction(12, 7)         # +6 can still fall short of it


def test_e4m3_encode_vs_torch(oracle_mod):
    vals = [float(v) for v in E4M3]
    mids = [(vals[i] + vals[i + 1]) / 2 for i in range(126)]
    rng = np.random.default_rng(11)
    xs = np.concatenate([
        _dense_around(mids + vals[1:], 64),
        rng.uniform(0, 464, 1 << 18).astype(np.float32),
        np.exp2(rng.uniform(-14, 8.85, 1 << 18)).astype(np.float32),
        np.array([0.0, 2.0 ** -10, 3 * 2.0 ** -11, 448.0, 463.99997], dtype=np.float32),
    ])
    xs = xs[(xs >= 0) & (xs < 464)]
    want = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle_mod.e4m3_encode(xs), want)


def test_e4m3_encode_saturates(oracle_mod):
    xs = np.array([448.0, 464.0, 470.0, 1e6, 3e38], dtype=np.float32)
    assert oracle_mod.e4m3_encode(xs).tolist() == [126] * 5


def _e2m1_from_bits(x32: np.ndarray) -> np.ndarray:
    """Third formulation, from the binary32 bit fields: below 1 the E2M1 grid is 0.5 apart, so
    the index is 2x rounded half-to-even (exact in float64); from 1 up, E2M1 keeps one mantissa
    bit, so the index is 2 + 2e + the top mantissa bit rounded half-to-even on the other 22
    bits (a carry moves to the next binade); 7 (the value 6) saturates everything above."""
    b = x32.view(np.uint32)
    e = (b >> 23).astype(np.int32) - 127
    keep = ((b >> 22) & 1).astype(np.int32)
    rest = b & 0x3FFFFF
    up = (rest > 0x200000) | ((rest == 0x200000) & (keep == 1))
    normal = np.minimum(2 + 2 * np.clip(e, 0, 3) + keep + up, 7)
    small = np.rint(x32.astype(np.float64) * 2.0)
    return np.where(x32 < 1.0, small, normal).astype(np.uint8)


def test_e2m1_every_binary32_in_0_16(oracle_mod):
    """Every non-negative binary32 below 16 (about 1.1e9 patterns): the oracle's midpoint ladder
    equals the bit-field formulation; the sign is handled apart (the index uses |x|)."""
    from concurrent.futures import ThreadPoolExecutor
    top = int(np.float32(16.0).view(np.uint32))
    step = 1 << 23

    def check(start):
        xs = np.arange(start, min(start + step, top), dtype=np.uint32).view(np.float32)
        got = oracle_mod.e2m1_index(xs)
        want = _e2m1_from_bits(xs)
        if np.array_equal(got, want):
            return None
        bad = np.nonzero(got != want)[0][:5]
        return f"mismatch at {xs[bad].tolist()}: {got[bad].tolist()} vs {want[bad].tolist()}"

    with ThreadPoolExecutor(max_workers=4) as pool:
        errors = [e for e in pool.map(check, range(0, top, step)) if e]
    assert not errors, errors[0]


def test_e4m3_encode_every_binary32_in_range(oracle_mod):
    """Every binary32 from 2^-10 (half the smallest subnormal code) up to 464 (half-way from 448
    to the next step; above it the oracle saturates, torch's conversion does not): the oracle's
    table scan equals torch's float8_e4m3fn conversion, a library routine, about 1.6e8 patterns;
    below 2^-10 everything encodes to 0."""
    from concurrent.futures import ThreadPoolExecutor
    lo = int(np.float32(2.0 ** -10).view(np.uint32))
    hi = int(np.float32(464.0).view(np.uint32))
    step = 1 << 22

    def check(start):
        xs = np.arange(start, min(start + step, hi), dtype=np.uint32).view(np.float32)
        got = oracle_mod.e4m3_encode(xs)
        want = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        if np.array_equal(got, want):
            return None
        bad = np.nonzero(got != want)[0][:5]
        return f"mismatch at {xs[bad].tolist()}: {got[bad].tolist()} vs {want[bad].tolist()}"

    with ThreadPoolExecutor(max_workers=8) as pool:
        errors = [e for e in pool.map(check, range(lo, hi, step)) if e]
    assert not errors, errors[0]
    tiny = np.arange(0, lo, 4099, dtype=np.uint32).view(np.float32)
    assert (oracle_mod.e4m3_encode(tiny) == 0).all()
