"""GPU parity of nvfp4_scale_search_rules: several rules in one call give, rule by rule, the
bytes of separate nvfp4_scale_search calls and of the oracle (paired launches for windows of
11 and 16 codes on bf16 W, single launches for the rest)."""
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


PAIRS = [[(0, -3, 7, False), (1, -8, 7, False)],      # the 8B attention modes
         [(1, -9, 6, False), (0, -3, 7, False)],
         [(1, -8, 7, False), (1, -9, 6, False)],
         [(0, -3, 7, False), (0, -5, 5, False)],
         [(1, -3, 7, False), (0, -8, 7, False)]]


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
