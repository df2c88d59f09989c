"""GPU parity of nvfp4_scale_search_rules: several rules in one call give, rule by rule, the
bytes of separate nvfp4_scale_search calls and of the oracle (paired launches for windows of
11 and 16 codes on bf16 W, scanned once where one 16-code window holds the other; one fused
launch for a 16-code window next to an exhaustive rule of the same objective; single launches
for the rest)."""
import numpy as np
import pytest
import torch

from block_scale_search_amd import workloads
from gpu_helpers import DEV, assert_same, oracle_search

pytestmark = pytest.mark.gpu


def _inputs(out, inp, dtype, seed, batch=None):
    W = workloads.normal_weights(out, inp, 0.02, 0.003, 25.0, seed, DEV, dtype, batch=batch)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 1)
    h = torch.exp(torch.randn((inp,) if batch is None else (batch, inp), generator=g,
                              device=DEV) * 2.0).float()
    return W, h


def _host(r):
    return {k: (None if v is None else v.cpu().numpy()) for k, v in r.items()}


def _check(nv, W, h, S, rules, what):
    fused = nv.scale_search_rules(W, h, S, rules)
    torch.cuda.synchronize()
    hn = h.cpu().numpy()
    Sn = S.cpu().numpy().reshape(-1)
    for (obj, lo, hi, exh), got in zip(rules, fused):
        hh = h if obj == nv.WMSE else None
        single = nv.scale_search(W, hh, S, obj, lo, hi, exh)
        torch.cuda.synchronize()
        g, s1 = _host(got), _host(single)
        for k in ("scales", "packed", "loss", "offset"):
            assert np.array_equal(g[k].view(np.uint8), s1[k].view(np.uint8)), f"{what} {k}"
        o = oracle_search(W, hn if obj == nv.WMSE else None, Sn if W.dim() == 3 else float(Sn[0]),
                          "wmse" if obj == nv.WMSE else "mse", lo, hi, exh)
        if W.dim() == 2:
            g = {k: v[None] for k, v in g.items()}
        assert_same(g, o, f"{what} rule ({obj}, {lo}, {hi}, {exh})")


PAIRS = [[(0, -3, 7, False), (1, -8, 7, False)],      # the 8B attention modes (nested windows)
         [(1, -9, 6, False), (0, -3, 7, False)],
         [(1, -8, 7, False), (1, -9, 6, False)],
         [(0, -3, 7, False), (0, -5, 5, False)],
         [(1, -3, 7, False), (0, -8, 7, False)],      # nested, MSE outside
         [(1, -9, 6, False), (0, -4, 6, False)],      # nested, the 11 codes ending at +6
         [(0, -8, 7, False), (1, -8, 7, False)],      # the same 16 codes, two objectives
         [(1, -8, 7, False), (1, -3, 7, False)]]      # nested, one objective


@pytest.mark.parametrize("rules", PAIRS, ids=lambda r: "+".join(f"{o}[{lo},{hi}]" for o, lo, hi, _ in r))
def test_pairs(nv, rules):
    W, h = _inputs(300, 272, torch.bfloat16, seed=41)
    S = nv.global_scale(W, nv.GS_AMAX_256)
    _check(nv, W, h, S, rules, "pair")


def test_unpaired_rules_and_odd_counts(nv):
    """An exhaustive rule, a 7-code window and a third rule run on their own, in order."""
    W, h = _inputs(129, 160, torch.bfloat16, seed=43)
    S = nv.global_scale(W, nv.GS_AMAX_448)
    _check(nv, W, h, S, [(0, -3, 7, False), (1, -8, 7, False), (1, 0, 0, True)], "three")
    _check(nv, W, h, S, [(1, 0, 0, True), (0, -3, 7, False), (1, -8, 7, False)], "exh first")
    _check(nv, W, h, S, [(0, -3, 3, False), (1, -9, 6, False)], "7-code window")
    _check(nv, W, h, S, [(1, -9, 6, False)], "one rule")


def test_fp32_weights_run_unpaired(nv):
    W, h = _inputs(67, 176, torch.float32, seed=45)
    S = nv.global_scale(W, nv.GS_AMAX_448)
    _check(nv, W, h, S, [(0, -3, 7, False), (1, -8, 7, False)], "fp32")


def test_batched_padded_rows(nv):
    base, h = _inputs(40, 256, torch.bfloat16, seed=47, batch=3)
    big = torch.full((3, 48, 320), 7.0, dtype=torch.bfloat16, device=DEV)
    big[:, :40, :256] = base
    view = big[:, :40, :256]
    S = nv.global_scale(view, nv.GS_AMAX_448)
    _check(nv, view, h, S, [(0, -3, 7, False), (1, -9, 6, False)], "batched")


def test_edge_groups(nv):
    """Zero groups, signed zeros and clipped windows at both ends of the code range."""
    W, h = _inputs(64, 512, torch.bfloat16, seed=49)
    W[0] = 0.0
    W[1, :16] = -0.0
    W[2, 16:32] = 1e-30
    W[3, 32:48] = 3e4
    h[:16] = 0.0
    S = nv.global_scale(W, nv.GS_AMAX_448)
    _check(nv, W, h, S, [(0, -3, 7, False), (1, -8, 7, False)], "edges")


def test_five_rules_two_pairs_and_clipped_windows(nv):
    """Five rules: two pairs and a single, on groups whose windows clip at code 1 and at 126."""
    W, h = _inputs(96, 320, torch.bfloat16, seed=51)
    W[0, :16] = 1e-30          # base code far below: windows clip at 1
    W[1, :16] = 2e4            # the tensor maximum: windows clip at 126 (rule 448)
    S = nv.global_scale(W, nv.GS_AMAX_448)
    rules = [(1, -8, 7, False), (0, -3, 7, False), (1, -9, 6, False), (1, -8, 7, False),
             (0, -5, 5, False)]
    _check(nv, W, h, S, rules, "five")


def _wide_range(out, inp, dtype, seed):
    """Rows scaled by 2^0 .. 2^-18 in turn, so that the groups' base codes run over the whole
    code range: windows clipped at 126, windows inside it, windows reaching the subnormal codes
    1..7 and clipped at 1."""
    W, h = _inputs(out, inp, dtype, seed)
    k = (torch.arange(out, device=DEV) % 19).float()
    W = (W.float() * torch.exp2(-k)[:, None]).to(dtype)
    return W, h


FUSED = [[(1, -9, 6, False), (1, 0, 0, True)],      # the 70B pair's two modes
         [(1, 0, 0, True), (1, -8, 7, False)],      # exhaustive rule first
         [(0, -15, 0, False), (0, 0, 0, True)],     # MSE, window ending at the base code
         [(0, 0, 15, False), (0, 0, 0, True)]]      # window starting at the base code


@pytest.mark.parametrize("rule", ["amax448", "amax256"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("rules", FUSED, ids=lambda r: "+".join(
    "exh" if e else f"{o}[{lo},{hi}]" for o, lo, hi, e in r))
def test_window_and_exhaustive_fused(nv, rules, dtype, rule):
    """A 16-code window beside an exhaustive rule of the same objective: one launch, whose two
    outputs equal the separate calls' and the oracle's, over base codes spanning 1..126."""
    W, h = _wide_range(152, 288, dtype, seed=53)
    W[0] = 0.0                       # zero groups
    W[1, :16] = -0.0
    S = nv.global_scale(W, nv.GS_AMAX_448 if rule == "amax448" else nv.GS_AMAX_256)
    _check(nv, W, h, S, rules, "fused")


def test_fused_overflow_negative_h_and_tiny_scale(nv):
    """The fused launch where losses overflow, where negative h, h = -0.0 or h above 2^100 turn
    the pruning off, and with a global scale whose lowest codes are subnormal (no octave
    identity)."""
    W, h = _inputs(48, 256, torch.float32, seed=55)
    W[:16] *= 1e4
    h[:64] = 3e38
    h[100:140] *= -1.0
    h[160:176] = -0.0
    h[192:200] = 2.0 ** 101
    S = nv.global_scale(W, nv.GS_AMAX_448)
    _check(nv, W, h, S, [(1, -9, 6, False), (1, 0, 0, True)], "fused overflow")
    Wt, ht = _inputs(32, 128, torch.float32, seed=57)
    Wt = Wt * 1e-33
    ht = ht * 1e30
    St = torch.tensor([2.6e-36], dtype=torch.float32, device=DEV)
    _check(nv, Wt, ht, St, [(1, -9, 6, False), (1, 0, 0, True)], "fused tiny S")
    _check(nv, Wt, ht, St, [(0, -8, 7, False), (0, 0, 0, True)], "fused tiny S mse")


def test_fused_batched_padded(nv):
    base, h = _inputs(40, 256, torch.bfloat16, seed=59, batch=3)
    big = torch.full((3, 48, 320), 7.0, dtype=torch.bfloat16, device=DEV)
    big[:, :40, :256] = base
    view = big[:, :40, :256]
    S = nv.global_scale(view, nv.GS_AMAX_256)
    _check(nv, view, h, S, [(1, -9, 6, False), (1, 0, 0, True)], "fused batched")


def test_scored_count(nv):
    """The exhaustive search's work count: at least the 16 centre codes and at most all 126 per
    group with a nonzero base code, all 126 where negative h turns the pruning off, and
    independent of what else the call runs."""
    W, h = _wide_range(152, 288, torch.bfloat16, seed=61)
    W[0] = 0.0
    S = nv.global_scale(W, nv.GS_AMAX_256)
    live = int((W.float().view(152, -1, 16).abs().amax(-1) > 0).sum())
    for obj in (nv.WMSE, nv.MSE):
        for lo in (-8, -9, 0, -15):
            n = nv.scale_search_scored(W, h, S, obj, lo)
            assert 16 * live <= n <= 126 * live, (obj, lo, n, live)
            assert n < 126 * live          # the bounds prune something on these weights
    neg = -h
    assert nv.scale_search_scored(W, neg, S, nv.WMSE, -8) == 126 * live
    assert nv.scale_search_scored(W, torch.full_like(h, -0.0), S, nv.WMSE, -8) == 126 * live
    # the count accumulates
    c = torch.full((1,), 5, dtype=torch.int64, device=DEV)
    nv.nvfp4_scale_search_scored(W, 1, 152, 288, 288, 0, 16, h, 0, nv.WMSE, -8, S, c)
    torch.cuda.synchronize()
    assert int(c.item()) == 5 + nv.scale_search_scored(W, h, S, nv.WMSE, -8)


@pytest.mark.parametrize("rules", [[(0, -3, 7, False), (1, -8, 7, False)],
                                   [(1, -8, 7, False), (0, -8, 7, False)]],
                         ids=["mse[-3,7]+wmse[-8,7]", "wmse[-8,7]+mse[-8,7]"])
def test_nested_windows_over_the_code_range(nv, rules):
    """Nested windows in one launch where waves mix unclipped, clipped and subnormal windows
    (those waves take the one-window-at-a-time path), against the separate calls and the
    oracle."""
    W, h = _wide_range(152, 288, torch.bfloat16, seed=63)
    W[0] = 0.0
    S = nv.global_scale(W, nv.GS_AMAX_448)
    _check(nv, W, h, S, rules, "nested wide range")
