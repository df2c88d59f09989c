"""GPU parity of on-line activation quantisation (ScaleSweep's WA / WAKV settings: the same
sweep on activations at inference time, with the dynamic per-tensor S = max|x| / (256 * 6)).

Bar: S, scale bytes and packed codes bit-identical to the oracle (global scale, then the
window search) and to the library's two-call path, from decode-sized batches to a prefill
chunk, for bf16 and f32 inputs, padded rows, and an all-zero tensor (S = 1, zero codes)."""
import numpy as np
import pytest
import torch

import oracle
from block_scale_search_amd import workloads
from gpu_helpers import DEV, host_w

pytestmark = pytest.mark.gpu


def _acts(T, inp, dtype, seed, ldx=None):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    sigma = torch.exp(torch.randn(inp, generator=g, device=DEV) * 1.5)
    ldx = ldx or inp
    x = torch.randn((T, ldx), generator=g, device=DEV)
    x[:, :inp] *= sigma
    return x.to(dtype)[:, :inp]


@pytest.mark.parametrize("T,inp,dtype,ldx", [(1, 4096, torch.bfloat16, None),
                                             (16, 4096, torch.bfloat16, None),
                                             (77, 1040, torch.float32, 1056),
                                             (2048, 4096, torch.bfloat16, 4104)])
def test_activations_match_oracle_and_two_call_path(nv, T, inp, dtype, ldx):
    X = _acts(T, inp, dtype, seed=T + inp, ldx=ldx)
    for rule, orule in ((nv.GS_AMAX_256, oracle.GS_AMAX_256), (nv.GS_AMAX_448, oracle.GS_AMAX_448)):
        for lo, hi in ((-3, 7), (0, 0), (-9, 6)):
            r = nv.quantize_activations(X, nv.MSE, lo, hi, rule)
            S2 = nv.global_scale(X, rule)
            q = nv.scale_search(X, None, S2, nv.MSE, lo, hi, with_stats=False)
            torch.cuda.synchronize()
            assert r["S"].item() == S2.item()
            assert torch.equal(r["scales"], q["scales"]) and torch.equal(r["packed"], q["packed"])
            Xh = host_w(X)
            S_o = oracle.global_scale(Xh, orule)
            assert r["S"].item() == np.float32(S_o)
            o = oracle.scale_search(Xh, None, oracle.MSE, lo, hi, False, S_o)
            np.testing.assert_array_equal(r["scales"].cpu().numpy(), o["scales"])
            np.testing.assert_array_equal(r["packed"].cpu().numpy(), o["packed"])


def test_activations_wmse_and_zero_tensor(nv):
    X = _acts(64, 512, torch.bfloat16, seed=5)
    h = torch.exp(torch.randn(512, device=DEV)).float()
    r = nv.quantize_activations(X, nv.WMSE, -8, 7, nv.GS_AMAX_256, h=h)
    S2 = nv.global_scale(X, nv.GS_AMAX_256)
    q = nv.scale_search(X, h, S2, nv.WMSE, -8, 7, with_stats=False)
    torch.cuda.synchronize()
    assert torch.equal(r["scales"], q["scales"]) and torch.equal(r["packed"], q["packed"])
    Z = torch.zeros((8, 256), dtype=torch.bfloat16, device=DEV)
    z = nv.quantize_activations(Z)
    torch.cuda.synchronize()
    assert z["S"].item() == 1.0
    assert (z["scales"] == 0).all() and (z["packed"] == 0).all()


def test_activations_prefill_chunk_of_8b_attention(nv):
    """The attention layer's calibration-shaped activations (8192 x 4096), sampled rows."""
    cfg = workloads.CONFIGS["attn8b"]
    X, _ = workloads.make_activation_chunk(cfg, workloads.make_sigma(cfg, DEV), 0, DEV)
    r = nv.quantize_activations(X)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 4095, 8191] + list(np.random.default_rng(9).choice(8192, 28, replace=False)))
    Xh = host_w(X)
    S_o = oracle.global_scale(Xh, oracle.GS_AMAX_256)
    assert r["S"].item() == np.float32(S_o)
    o = oracle.scale_search(Xh[rows], None, oracle.MSE, -3, 7, False, S_o)
    np.testing.assert_array_equal(r["scales"].cpu().numpy()[rows], o["scales"])
    np.testing.assert_array_equal(r["packed"].cpu().numpy()[rows], o["packed"])


@pytest.mark.parametrize("T", [64, 4096])      # the fused path and the three-kernel path
def test_activations_without_s_output(nv, T):
    """S_out = NULL: S stays in the workspace; codes equal those of the path that returns S."""
    X = _acts(T, 4096, torch.bfloat16, seed=T)
    r = nv.quantize_activations(X)
    sc = torch.empty_like(r["scales"])
    pk = torch.empty_like(r["packed"])
    ws = torch.empty(nv.nvfp4_quantize_activations_workspace_size(T, 4096), dtype=torch.uint8,
                     device=DEV)
    nv.nvfp4_quantize_activations(X, T, 4096, 4096, nv.MSE, None, -3, 7, nv.GS_AMAX_256, None,
                                  sc, pk, ws)
    torch.cuda.synchronize()
    assert torch.equal(sc, r["scales"]) and torch.equal(pk, r["packed"])
