"""GPU parity of the proposal-centred search (Replay the Curvature §4.1.3-§4.1.4, App. D.2): a
window around a per-group proposal code plus the incoming code, which is kept on ties.

Bar: scale bytes, packed codes, offsets and losses bit-exact against the oracle, on
ragged shapes, a batch with per-matrix S, proposals outside 1..126, windows that clip at both
ends of the code range, with and without incoming codes, and all-equal losses (h = 0)."""
import numpy as np
import pytest
import torch

import oracle
from block_scale_search_amd import workloads
from gpu_helpers import DEV, OBJ, assert_same, host_w

pytestmark = pytest.mark.gpu


def _inputs(batch, out, inp, dtype, seed):
    W = workloads.normal_weights(out, inp, 0.02, 0.004, 25.0, seed, DEV, dtype, batch=batch)
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 1)
    h = torch.exp(torch.randn((batch, inp), generator=g, device=DEV) * 2.5).float()
    return W, h, g


def _codes(nv, W, S, g, spread, incoming_kind):
    """Proposal codes around the base codes (some outside 1..126) and incoming codes."""
    base = nv.scale_search(W, None, S, nv.MSE, 0, 0, with_stats=False)["scales"].to(torch.int32)
    off = torch.randint(-spread, spread + 1, base.shape, generator=g, device=DEV, dtype=torch.int32)
    center = (base + off).clamp(0, 255)
    center.view(-1)[::37] = 0                                    # below the code range
    center.view(-1)[5::41] = 200                                 # above it
    center = center.to(torch.uint8).contiguous()
    if incoming_kind == "none":
        return center, None
    if incoming_kind == "base":
        return center, base.to(torch.uint8).contiguous()
    inc = torch.randint(0, 140, base.shape, generator=g, device=DEV, dtype=torch.int32)  # some invalid
    return center, inc.to(torch.uint8).contiguous()


def _oracle(W, h, S, obj, lo, hi, center, incoming):
    Wn = host_w(W)
    c = center.cpu().numpy()
    i = None if incoming is None else incoming.cpu().numpy()
    res = [oracle.scale_search_proposal(Wn[b], None if h is None else h[b].cpu().numpy(), OBJ[obj],
                                        lo, hi, c[b], None if i is None else i[b], float(S[b]))
           for b in range(Wn.shape[0])]
    return {k: np.stack([r[k] for r in res]) for k in res[0]}


def _gpu(nv, W, h, S, obj, lo, hi, center, incoming):
    r = nv.scale_search_proposal(W, h, S, nv.WMSE if obj == "wmse" else nv.MSE, center, incoming,
                                 lo, hi)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in r.items()}


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("incoming_kind", ["none", "base", "random"])
def test_proposal_parity(nv, dtype, incoming_kind):
    W, h, g = _inputs(2, 77, 336, dtype, seed=91)
    S = nv.global_scale(W, nv.GS_AMAX_448)
    S_h = S.cpu().numpy()
    center, incoming = _codes(nv, W, S, g, 6, incoming_kind)
    for obj, lo, hi in (("wmse", -4, 4), ("mse", -4, 4), ("wmse", -9, 6), ("mse", -3, 7),
                        ("wmse", 0, 0), ("wmse", -2, 12)):
        gg = _gpu(nv, W, h if obj == "wmse" else None, S, obj, lo, hi, center, incoming)
        o = _oracle(W, h if obj == "wmse" else None, S_h, obj, lo, hi, center, incoming)
        assert_same(gg, o, f"proposal {obj} [{lo},{hi}] incoming={incoming_kind} {dtype}")


def test_proposal_edges_and_ties(nv):
    """Proposals at the bottom and top of the code range (clipped windows, subnormal codes),
    tiny and zero groups, and h = 0 (every loss 0: the incoming code must be kept)."""
    W, h, g = _inputs(1, 64, 256, torch.float32, seed=93)
    W[0, 0, :32] = 0.0
    W[0, 1] *= 1e-4
    W[0, 2, 16:32] = torch.linspace(-3.0, 3.0, 16, device=DEV)
    S = nv.global_scale(W, nv.GS_AMAX_448)
    S_h = S.cpu().numpy()
    shape = (1, 64, 16)
    bottom = torch.randint(0, 10, shape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    top = torch.randint(118, 130, shape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    inc = torch.randint(1, 127, shape, generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    for center in (bottom, top):
        for hh in (h, torch.zeros_like(h)):
            for incoming in (None, inc):
                gg = _gpu(nv, W, hh, S, "wmse", -4, 4, center, incoming)
                o = _oracle(W, hh, S_h, "wmse", -4, 4, center, incoming)
                assert_same(gg, o, "proposal edges")
    # h = 0: the incoming code wins every non-zero group
    gg = _gpu(nv, W, torch.zeros_like(h), S, "wmse", -4, 4, top, inc)
    nz = (W[0].abs().reshape(64, 16, 16).amax(-1) > 0).cpu().numpy()
    assert (gg["scales"][0][nz] == inc[0].cpu().numpy()[nz]).all()


def test_proposal_at_base_equals_window_search(nv):
    """Centred on the base code with no incoming code, the proposal search is the plain window
    search, bit for bit, on the GPU too."""
    W, h, g = _inputs(1, 96, 512, torch.bfloat16, seed=95)
    S = nv.global_scale(W, nv.GS_AMAX_448)
    base = nv.scale_search(W, None, S, nv.MSE, 0, 0, with_stats=False)["scales"].contiguous()
    for obj, lo, hi in (("wmse", -4, 4), ("wmse", -8, 7), ("mse", -3, 7)):
        p = _gpu(nv, W, h if obj == "wmse" else None, S, obj, lo, hi, base, None)
        q = nv.scale_search(W, h if obj == "wmse" else None, S, nv.WMSE if obj == "wmse" else nv.MSE,
                            lo, hi)
        torch.cuda.synchronize()
        for k in ("scales", "packed", "loss", "offset"):
            np.testing.assert_array_equal(p[k], q[k].cpu().numpy(), err_msg=f"{obj} {k}")
