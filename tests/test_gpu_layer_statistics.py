"""GPU parity of the fused layer statistics (h of X and S of W in two launches): bit-identical
to nvfp4_diag_hessian followed by nvfp4_global_scale, and against the oracle (h within 1e-5
relative, S exact).

Cases: bf16 and f32 X and W in all four pairings, ragged token and column counts, X above the
256 MiB size where the h pass switches to 4-wave workgroups, strided rows, accumulation into a
running sum, empty token chunks, an all-zero W (S = 1), both global-scale rules, and the full
8B-shaped layers as the bench step runs them."""
import numpy as np
import pytest
import torch

import oracle
from block_scale_search_amd import workloads
from gpu_helpers import DEV, host_w

pytestmark = pytest.mark.gpu

H_RTOL = 1e-5


def _x(T, inp, dtype, seed):
    sig = workloads.channel_sigma(inp, 1.5, seed=inp + seed, device=DEV)
    return workloads.activations(T, sig, seed=seed, device=DEV, dtype=dtype)


def _w(out, inp, dtype, seed):
    return workloads.normal_weights(out, inp, 0.02, 0.003, 25.0, seed, DEV, dtype)


def _two_calls(nv, X, W, rule, acc=None, accumulate=False):
    a = None if acc is None else acc.clone()
    acc2, h2 = nv.diag_hessian(X, a, accumulate=accumulate)
    S2 = nv.global_scale(W, rule)
    return acc2, h2, S2


def _check(nv, X, W, rule, acc=None, accumulate=False):
    a = None if acc is None else acc.clone()
    acc1, h1, S1 = nv.layer_statistics(X, W, rule, a, accumulate)
    acc2, h2, S2 = _two_calls(nv, X, W, rule, acc, accumulate)
    torch.cuda.synchronize()
    assert torch.equal(acc1, acc2), "h_acc differs from nvfp4_diag_hessian"
    assert torch.equal(h1.view(torch.int32), h2.view(torch.int32)), "h differs"
    assert torch.equal(S1.view(torch.int32), S2.view(torch.int32)), "S differs"
    return acc1, h1, S1


@pytest.mark.parametrize("xd", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("wd", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T,inp,out", [(1, 16, 1), (513, 1000 // 16 * 16, 37), (3000, 4096, 300)])
def test_matches_two_calls_and_oracle(nv, xd, wd, T, inp, out):
    X = _x(T, inp, xd, seed=T)
    W = _w(out, inp, wd, seed=out)
    for rule, orule in ((nv.GS_AMAX_448, oracle.GS_AMAX_448), (nv.GS_AMAX_256, oracle.GS_AMAX_256)):
        acc, h, S = _check(nv, X, W, rule)
        acc_o, h_o = oracle.diag_hessian(host_w(X))
        np.testing.assert_allclose(acc.cpu().numpy(), acc_o, rtol=1e-12, atol=0)
        np.testing.assert_allclose(h.cpu().numpy(), h_o, rtol=H_RTOL, atol=0)
        assert S.item() == np.float32(oracle.global_scale(host_w(W), orule))


def test_wide_x_and_strided_rows(nv):
    """X of 288 MiB (4-wave h workgroups), X and W as column slices of wider buffers."""
    Xb = _x(36864, 4160, torch.bfloat16, seed=5)
    X = Xb[:, :4096]
    Wb = _w(1024, 4160, torch.bfloat16, seed=6)
    W = Wb[:, :4096]
    _check(nv, X, W, nv.GS_AMAX_256)


def test_accumulate_empty_chunk_and_zero_weights(nv):
    X = _x(700, 640, torch.bfloat16, seed=7)
    W = _w(64, 640, torch.float32, seed=8)
    acc, _, _ = _check(nv, X, W, nv.GS_AMAX_448)
    acc2, _, _ = _check(nv, X, W, nv.GS_AMAX_448, acc=acc, accumulate=True)
    acc_o, _ = oracle.diag_hessian(host_w(X))
    acc_o, _ = oracle.diag_hessian(host_w(X), acc_o)
    np.testing.assert_allclose(acc2.cpu().numpy(), acc_o, rtol=1e-12, atol=0)
    # an empty token chunk keeps the running sum; an all-zero W gives S = 1
    Wz = torch.zeros_like(W)
    acc3, _, S = _check(nv, X[:0], Wz, nv.GS_AMAX_256, acc=acc2, accumulate=True)
    assert torch.equal(acc3, acc2) and S.item() == 1.0


@pytest.mark.parametrize("name", ["attn8b", "down8b"])
def test_full_size_workloads(nv, name):
    """The one-chunk workloads as the bench step runs them: bit-identical to the two calls, S
    equal to the oracle's, h against the oracle on a sampled column block."""
    cfg = workloads.CONFIGS[name]
    W = workloads.make_weights(cfg, DEV)
    sig = workloads.make_sigma(cfg, DEV)
    X, _ = workloads.make_activation_chunk(cfg, sig, 0, DEV)
    rule = nv.GS_AMAX_256 if cfg.gs_rule == "amax256" else nv.GS_AMAX_448
    orule = oracle.GS_AMAX_256 if cfg.gs_rule == "amax256" else oracle.GS_AMAX_448
    acc, h, S = _check(nv, X, W, rule)
    assert S.item() == np.float32(oracle.global_scale(host_w(W), orule))
    cols = slice(1024, 1024 + 256)
    acc_o, h_o = oracle.diag_hessian(host_w(X[:, cols].contiguous()))
    np.testing.assert_allclose(h[cols].cpu().numpy(), h_o, rtol=H_RTOL, atol=0)
    np.testing.assert_allclose(acc[cols].cpu().numpy(), acc_o, rtol=1e-12, atol=0)
