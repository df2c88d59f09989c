"""The E2M1 rounding that every kernel takes from the hardware conversion, pinned on the GPU.

The kernels round to E2M1 with gfx950's down-conversion to fp4 (and its exact up-conversion).
The format fixes round-to-nearest, ties to the even code, no infinity (values above 6 become 6)
(ScaleSweep technical summary, Problem Statement: FP4 E2M1 values; Replay the Curvature
summary, §4.1.1: normalised values rounded to the E2M1 levels). Two paths use the conversion:

* scale operand 1.0: the pack kernel, the search's single codes and the final re-quantisation.
  `test_pack_rounds_every_finite_binary32` runs nvfp4_pack with S = 1 and scale byte 56, whose
  effective scale is exactly 1 (E4M3 code 56 = 2^0), so the kernel converts w itself; it covers
  every finite binary32 of both signs (zeros and subnormals included, 2^32 - 2^24 values) and
  compares every nibble with the oracle's pack of the same values.
* scale operand 2.0: the octave-paired search, which converts x = |w| r[c] once at scale 1 for
  code c and once at scale 2 (x / 2) for code c + 8. `test_octave_pairs_on_midpoints` builds
  groups whose magnitudes sit exactly on E2M1 midpoints (and one ulp either side) of the upper
  code of a pair, so that the scale-2 conversion sees the ties, and compares scales, codes,
  offsets and loss bits with the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import DEV, assert_same, gpu_search, host_w, oracle_search

pytestmark = pytest.mark.gpu

MIDPOINTS = (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)
CODE_ONE = 56          # E4M3 0x38 = 2^(7-7) * (1 + 0/8) = 1.0


def test_tie_table_through_pack(nv):
    """The E2M1 ties and saturation, value by value, at an effective scale of exactly 1."""
    x = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 6.5, 7.0, 1e30, 0.0,
                      -0.25, -0.75, -1.25, -1.75, -2.5, -3.5, -5.0, -6.0, -6.5, -7.0, -1e30, -0.0,
                      0.2499999, 0.2500001, 5.0000005, 4.9999995, 1e-45, -1e-45, 0.5, 3.0],
                     dtype=torch.float32, device=DEV).reshape(2, 16)
    p = nv.pack(x, torch.full((2, 1), CODE_ONE, dtype=torch.uint8, device=DEV),
                torch.ones(1, device=DEV)).cpu().numpy()
    nib = oracle.unpack_nibbles(p).reshape(-1)
    # even-index ties: 0.25->0, 0.75->1 (idx 2), 1.25->1 (2), 1.75->2 (4), 2.5->2 (4),
    # 3.5->4 (6), 5->4 (6); 6 and above -> 6 (7); the sign bit is kept, also for zero
    want_pos = [0, 2, 2, 4, 4, 6, 6, 7, 7, 7, 7, 0]
    want = want_pos + [8 | v for v in want_pos] + [0, 1, 7, 6, 0, 8, 1, 5]
    assert nib.tolist() == want


def test_pack_rounds_every_finite_binary32(nv):
    """Every finite binary32 w of both signs, packed at S = 1 and scale byte 56 (x = w exactly),
    against the oracle's pack of the same values, nibble by nibble."""
    inp = 4096
    end = 0x7F800000                       # first non-finite pattern (+inf)
    chunk = 1 << 28
    ones = torch.ones(1, device=DEV)
    checked = 0
    for start in range(0, end, chunk):
        stop = min(end, start + chunk)
        rows = (stop - start) // inp
        print(f"binary32 patterns {start:#010x}..{stop - 1:#010x}", flush=True)
        bits = torch.arange(start, stop, dtype=torch.int64, device=DEV).to(torch.int32)
        W = bits.view(torch.float32).reshape(rows, inp)
        scales = torch.full((rows, inp // 16), CODE_ONE, dtype=torch.uint8, device=DEV)
        p_pos = nv.pack(W, scales, ones).cpu().numpy()
        p_neg = nv.pack(torch.neg(W), scales, ones).cpu().numpy()
        del W, bits
        Wn = np.arange(start, stop, dtype=np.uint32).view(np.float32).reshape(rows, inp)
        sc = np.full((rows, inp // 16), CODE_ONE, dtype=np.uint8)
        o_pos = oracle.pack(Wn, sc, 1.0)
        bad = np.flatnonzero(p_pos != o_pos)
        assert bad.size == 0, f"positive: {bad.size} bytes differ, first at pattern " \
                              f"{start + 2 * int(bad[0]):#010x}"
        o_neg = oracle.pack(np.negative(Wn), sc, 1.0)
        bad = np.flatnonzero(p_neg != o_neg)
        assert bad.size == 0, f"negative: {bad.size} bytes differ, first at pattern " \
                              f"{start + 2 * int(bad[0]):#010x}"
        checked += 2 * (stop - start)
    assert checked == 2 * end
    print(f"{checked} finite binary32 values rounded identically", flush=True)


def _midpoint_layer(out, groups, S, seed, dtype, near):
    """Groups whose first element fixes the base code b (|w| = 6 eff(b), so fl(amax/6)/S is
    exactly E4M3(b)), and whose other elements sit on E2M1 midpoints (or one ulp off, if
    `near`) of a random code c in b-1 .. b+7 with S a power of two, so that x = |w| r[c - 8]
    equals twice a midpoint and the scale-2 conversion of the pair (c - 8, c) sees the tie.
    Base codes lie in 17 .. 119, so every window of the tests stays in the normal codes."""
    rng = np.random.default_rng(seed)
    inp = 16 * groups
    W = np.zeros((out, inp), dtype=np.float32)
    for o in range(out):
        for g in range(groups):
            b = int(rng.integers(17, 120))
            amax = np.float32(6.0 * oracle.e4m3_value(b) * S)
            v = np.empty(16, dtype=np.float32)
            v[0] = amax
            for j in range(1, 16):
                while True:
                    c = b + int(rng.integers(-1, 8))
                    m = float(rng.choice(MIDPOINTS))
                    x = np.float32(m * oracle.e4m3_value(c) * S)
                    if x <= amax:
                        break
                if near and rng.random() < 0.5:
                    x = np.nextafter(x, np.float32(np.inf) if rng.random() < 0.5 else np.float32(0))
                v[j] = x
            rng.shuffle(v)
            v *= np.where(rng.random(16) < 0.5, -1.0, 1.0).astype(np.float32)
            W[o, 16 * g:16 * g + 16] = v
    Wt = torch.from_numpy(W).to(DEV)
    if dtype == torch.bfloat16:
        # every value is exact in bf16 (at most 7 significant bits); the one-ulp neighbours
        # are taken in bf16 instead (adding -1, 0 or 1 to the bit pattern of a finite non-zero
        # bf16 moves its magnitude by at most one ulp)
        Wb = Wt.to(torch.bfloat16)
        assert near or torch.equal(Wb.float(), Wt)
        if near:
            step = torch.from_numpy(rng.integers(-1, 2, W.shape).astype(np.int16)).to(DEV)
            Wb = (Wb.view(torch.int16) + step).view(torch.bfloat16)
        return Wb
    return Wt


def _ties_on_scale2(W: torch.Tensor, S: float, window):
    """How many (element, pair) conversions at scale 2 of the window's octave pairs land exactly
    on an E2M1 midpoint, recomputed on the host in binary32."""
    lo, hi = window
    eff, rcp = oracle.scale_tables(S)
    Wn = W.float().abs().cpu().numpy().reshape(-1, 16)
    base = oracle.e4m3_encode((Wn.max(axis=1) / np.float32(6.0)) / np.float32(S)).astype(np.int64)
    base = np.maximum(base, 1)
    n = hi - lo + 1
    pairs = min(8, max(0, n - 8))
    mids = np.array(MIDPOINTS, dtype=np.float32)
    ties = 0
    for p in range(pairs):
        c_lo = np.clip(base + lo + p, 1, 126)
        x = Wn * rcp[c_lo][:, None]
        ties += int(np.isin(x / np.float32(2.0), mids).sum())
    return ties


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("near", [False, True])
def test_octave_pairs_on_midpoints(nv, dtype, near):
    """The paired search on magnitudes at E2M1 midpoints of the pairs' upper codes: WMSE
    [-9,6], MSE [-3,7] and WMSE [-8,7] alone, and MSE [-3,7] + WMSE [-8,7] as one paired
    launch (bf16), each against the oracle bit for bit (losses included)."""
    S = 2.0 ** -10
    W = _midpoint_layer(96, 24, S, seed=11 + int(near) + (2 if dtype == torch.bfloat16 else 0),
                        dtype=dtype, near=near)
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    h = torch.exp(torch.randn(W.shape[1], generator=g, device=DEV) * 1.5).float()
    hn = h.cpu().numpy()
    St = torch.tensor([S], dtype=torch.float32, device=DEV)
    windows = [("wmse", -9, 6), ("mse", -3, 7), ("wmse", -8, 7)]
    for obj, lo, hi in windows:
        gg = gpu_search(nv, W, h if obj == "wmse" else None, St, obj, lo, hi, False)
        o = oracle_search(W, hn if obj == "wmse" else None, S, obj, lo, hi, False)
        assert_same(gg, o, f"{obj} [{lo},{hi}] {dtype} near={near}")
        ties = _ties_on_scale2(W, S, (lo, hi))
        print(f"{obj} [{lo},{hi}] {dtype} near={near}: {ties} scale-2 conversions on a midpoint",
              flush=True)
        if not near:
            assert ties > 1000
    if dtype == torch.bfloat16:
        rules = [(nv.MSE, -3, 7, False), (nv.WMSE, -8, 7, False)]
        res = nv.scale_search_rules(W, h, St, rules)
        torch.cuda.synchronize()
        for (obj, lo, hi, _), r in zip(rules, res):
            name = "wmse" if obj == nv.WMSE else "mse"
            o = oracle_search(W, hn if name == "wmse" else None, S, name, lo, hi, False)
            assert_same({k: v.cpu().numpy()[None] for k, v in r.items()}, o,
                        f"paired launch {name} [{lo},{hi}] near={near}")


def test_midpoints_on_subnormal_and_clipped_codes(nv):
    """Midpoint magnitudes where the windows reach the subnormal codes 1..7 and the top code
    126 (the per-code path, scale 1.0 only), against the oracle."""
    rng = np.random.default_rng(21)
    out, groups = 64, 16
    W = np.zeros((out, 16 * groups), dtype=np.float32)
    S = 2.0 ** -12
    for o in range(out):
        for g in range(groups):
            b = int(rng.choice([1, 2, 3, 5, 7, 9, 12, 120, 123, 125, 126]))
            v = np.array([float(rng.choice(MIDPOINTS)) * oracle.e4m3_value(
                min(126, max(1, b + int(rng.integers(-3, 4))))) * S for _ in range(16)],
                dtype=np.float32)
            v *= np.where(rng.random(16) < 0.5, -1.0, 1.0).astype(np.float32)
            W[o, 16 * g:16 * g + 16] = v
    Wt = torch.from_numpy(W).to(DEV)
    St = torch.tensor([S], dtype=torch.float32, device=DEV)
    h = torch.ones(W.shape[1], device=DEV)
    for obj, lo, hi in [("wmse", -9, 6), ("mse", -3, 7)]:
        gg = gpu_search(nv, Wt, h if obj == "wmse" else None, St, obj, lo, hi, False)
        o = oracle_search(Wt, h.cpu().numpy() if obj == "wmse" else None, S, obj, lo, hi, False)
        assert_same(gg, o, f"{obj} [{lo},{hi}] subnormal/clipped")
    gg = gpu_search(nv, Wt, h, St, "wmse", 0, 0, True)
    o = oracle_search(Wt, h.cpu().numpy(), S, "wmse", 0, 0, True)
    assert_same(gg, o, "exhaustive subnormal/clipped")
