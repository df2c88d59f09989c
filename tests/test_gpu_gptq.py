"""GPU parity of GPTQ with the window search as local quantiser (H-Scale App. B; Replay the
Curvature §3): scale bytes, packed codes and the final binary32 weights bit-exact against the
oracle's sequential implementation, given the same inverse-Hessian factor U.

Cases: inner blocks of 64 columns with a ragged last block (in = 208), several outer blocks of
256 with a ragged last one (in = 592: 256 + 256 + 64 + 16), rows off the 16-row and 128-row
tiles, bf16 and f32 W, WMSE and MSE windows, a wide window clipped at codes 1 and 126 (scored
16 codes per pass), a one-code window, all-zero groups and negative zeros, the identity factor
(no propagation), a Hessian from correlated activations (strong propagation), and the full
8B-shaped layers (4096 x 4096 and 4096 x 14336) checked on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
from block_scale_search_amd import workloads
from gpu_helpers import DEV, host_w

pytestmark = pytest.mark.gpu


def _factor(X, damp=0.01):
    H = X.astype(np.float64).T @ X.astype(np.float64)
    H += damp * np.mean(np.diag(H)) * np.eye(H.shape[0])
    L = np.linalg.cholesky(np.linalg.inv(H))
    return L.T.astype(np.float32), np.diag(H).astype(np.float32)


def _case(out, inp, dtype, seed, T=512):
    rng = np.random.default_rng(seed)
    W = workloads.normal_weights(out, inp, 0.02, 0.01, 15.0, seed, DEV, dtype)
    A = rng.standard_normal((inp, inp)) * 0.3 + np.eye(inp)
    X = (rng.standard_normal((T, inp)) @ A * np.exp(rng.standard_normal(inp) * 0.7)).astype(np.float32)
    U, h = _factor(X)
    return W, U, h


def _compare(nv, W, U, h, obj, lo, hi):
    S = nv.global_scale(W, nv.GS_AMAX_448)
    Ud = torch.from_numpy(U).to(DEV)
    hd = torch.from_numpy(h).to(DEV)
    g = nv.gptq(W, Ud, hd if obj == "wmse" else None, S,
                nv.WMSE if obj == "wmse" else nv.MSE, lo, hi, with_final=True)
    torch.cuda.synchronize()
    o = oracle.gptq(host_w(W), U, h if obj == "wmse" else None,
                    oracle.WMSE if obj == "wmse" else oracle.MSE, lo, hi, float(S.item()))
    for k in ("scales", "packed"):
        bad = np.argwhere(g[k].cpu().numpy() != o[k])
        assert bad.size == 0, f"{k}: {len(bad)} mismatches, first {bad[:3].tolist()}"
    wf = g["W_final"].cpu().numpy()
    bad = np.argwhere(wf.view(np.uint32) != o["W_final"].view(np.uint32))
    assert bad.size == 0, f"W_final: {len(bad)} mismatches, first {bad[:3].tolist()}"


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("obj,lo,hi", [("wmse", -9, 6), ("mse", -3, 7), ("wmse", -2, 2)])
def test_gptq_parity(nv, dtype, obj, lo, hi):
    W, U, h = _case(100, 208, dtype, seed=201)
    _compare(nv, W, U, h, obj, lo, hi)


def test_gptq_identity_factor_equals_window_search(nv):
    W, _, h = _case(70, 192, torch.bfloat16, seed=203)
    U = np.eye(192, dtype=np.float32)
    _compare(nv, W, U, h, "wmse", -8, 7)
    S = nv.global_scale(W, nv.GS_AMAX_448)
    g = nv.gptq(W, torch.from_numpy(U).to(DEV), torch.from_numpy(h).to(DEV), S)
    q = nv.scale_search(W, torch.from_numpy(h).to(DEV), S, nv.WMSE, -9, 6)
    torch.cuda.synchronize()
    assert torch.equal(g["scales"], q["scales"]) and torch.equal(g["packed"], q["packed"])


def test_gptq_larger_layer(nv):
    """512 rows x 1024 columns (16 blocks), bf16."""
    W, U, h = _case(512, 1024, torch.bfloat16, seed=205, T=2048)
    _compare(nv, W, U, h, "wmse", -9, 6)


@pytest.mark.parametrize("lo,hi", [(-9, 6), (-30, 25), (0, 0)])
def test_gptq_outer_blocks_ragged(nv, lo, hi):
    """592 columns (two outer blocks of 256, then 64 + 16), 37 rows."""
    W, U, h = _case(37, 592, torch.bfloat16, seed=207, T=1024)
    _compare(nv, W, U, h, "wmse", lo, hi)


def test_gptq_zero_groups_and_negative_zeros(nv):
    """Rows and groups of zeros (code 0) and negative zeros, f32, MSE and WMSE."""
    W, U, h = _case(40, 272, torch.float32, seed=209)
    W[3] = 0.0
    W[5, 16:32] = -0.0
    W[7, 0:16] = 0.0
    W[7, 3] = -0.0
    W[9, 256:272] = 0.0
    _compare(nv, W, U, h, "wmse", -9, 6)
    _compare(nv, W, U, h, "mse", -3, 7)


def _workload_factor(cfg, W):
    """U and h of a workload's first activation chunk, as bench.py builds them (binary64 Gram
    matrix on the GPU, damping 0.01 mean(diag), Cholesky factor of the inverse)."""
    sig = workloads.make_sigma(cfg, DEV)
    X, _ = workloads.make_activation_chunk(cfg, sig, 0, DEV)
    Xd = X.double()
    H = Xd.T @ Xd
    del Xd, X
    H += 0.01 * torch.diagonal(H).mean() * torch.eye(cfg.inp, dtype=torch.float64, device=DEV)
    U = torch.linalg.cholesky(torch.cholesky_inverse(torch.linalg.cholesky(H))).T.contiguous()
    return U.float().contiguous(), torch.diagonal(H).float().contiguous()


@pytest.mark.parametrize("name,lo,hi", [("attn8b", -8, 7), ("down8b", -9, 6)])
def test_gptq_full_size_sampled_rows(nv, name, lo, hi):
    """Full 8B-shaped layers on the GPU; rows are independent, so sampled rows (first, last and
    seeded ones) are checked bit-exact against the oracle run on those rows alone."""
    cfg = workloads.CONFIGS[name]
    W = workloads.make_weights(cfg, DEV)
    U, h = _workload_factor(cfg, W)
    S = nv.global_scale(W, nv.GS_AMAX_256 if cfg.gs_rule == "amax256" else nv.GS_AMAX_448)
    g = nv.gptq(W, U, h, S, nv.WMSE, lo, hi, with_final=True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, cfg.out - 1], rng.choice(cfg.out, 29, replace=False)]))
    o = oracle.gptq(host_w(W[torch.from_numpy(rows).to(DEV)]), U.cpu().numpy(), h.cpu().numpy(),
                    oracle.WMSE, lo, hi, float(S.item()))
    for k in ("scales", "packed"):
        got = g[k][torch.from_numpy(rows).to(DEV)].cpu().numpy()
        bad = np.argwhere(got != o[k])
        assert bad.size == 0, f"{name} {k}: {len(bad)} mismatches, first {bad[:3].tolist()}"
    wf = g["W_final"][torch.from_numpy(rows).to(DEV)].cpu().numpy()
    bad = np.argwhere(wf.view(np.uint32) != o["W_final"].view(np.uint32))
    assert bad.size == 0, f"{name} W_final: {len(bad)} mismatches, first {bad[:3].tolist()}"


@pytest.mark.parametrize("out,inp", [(1, 16), (3, 48), (17, 64), (16, 80)])
def test_gptq_small_shapes(nv, out, inp):
    """One group, partial inner blocks and single rows."""
    W, U, h = _case(out, inp, torch.bfloat16, seed=211 + inp, T=256)
    _compare(nv, W, U, h, "wmse", -9, 6)
