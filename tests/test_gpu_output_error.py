"""GPU parity of the layer-output error (H-Scale §3: layer-output reconstruction criterion).

err[o] = sum_t (sum_i x_ti (w_oi - w_hat_oi))^2 against the oracle's binary64 value.
Tolerance: 1e-4 relative per row. The GPU splits E = fl(w - w_hat) into bf16 E_hi + E_lo
(relative representation error <= 2^-17), multiplies exactly in binary32 on MFMA and
accumulates in binary32 over `in` terms (error ~ sqrt(in) 2^-24 of sum |x e|); squaring and
summing over tokens averages these independent errors. Rows whose residual is exactly zero
must give exactly zero.
"""
import numpy as np
import pytest
import torch

import oracle
from block_scale_search_amd import workloads
from gpu_helpers import DEV, host_w

pytestmark = pytest.mark.gpu

RTOL = 1e-4


def _case(T, out, inp, w_dtype, seed, ldx=None):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    W = workloads.normal_weights(out, inp, 0.02, 0.004, 25.0, seed, DEV, w_dtype)
    sigma = torch.exp(torch.randn(inp, generator=g, device=DEV) * 1.2)
    ldx = ldx or inp
    Xbuf = torch.randn((T, ldx), generator=g, device=DEV) * torch.nn.functional.pad(sigma, (0, ldx - inp), value=1.0)
    X = Xbuf.to(torch.bfloat16)[:, :inp]
    return W, X


def _check(nv, X, W, S, packed, scales, rows=None, what=""):
    err = nv.output_error(X, W, packed, scales, S)
    torch.cuda.synchronize()
    e = err.cpu().numpy()
    if rows is None:
        rows = np.arange(W.shape[0])
    r_t = torch.from_numpy(rows).to(DEV)
    o = oracle.output_error(host_w(X), host_w(W[r_t]), packed[r_t].cpu().numpy(),
                            scales[r_t].cpu().numpy(), float(S.item()))
    np.testing.assert_allclose(e[rows], o, rtol=RTOL, atol=0, err_msg=what)
    return e, o


@pytest.mark.parametrize("w_dtype", [torch.bfloat16, torch.float32])
def test_output_error_ragged(nv, w_dtype):
    """Token count, row count and column count off the 256/256/32 tiles; padded X rows."""
    W, X = _case(300, 150, 272, w_dtype, seed=101, ldx=280)
    W[5] = 0.0                                                   # a zero row: exactly 0
    S = nv.global_scale(W, nv.GS_AMAX_448)
    for lo, hi in ((0, 0), (-9, 6)):
        r = nv.scale_search(W, None, S, nv.MSE, lo, hi, with_stats=False)
        e, o = _check(nv, X, W, S, r["packed"], r["scales"], what=f"[{lo},{hi}] {w_dtype}")
        assert e[5] == 0.0


@pytest.mark.parametrize("T,out,inp", [(700, 600, 1040), (1024, 2048, 256), (256, 256, 32)])
def test_output_error_tiles(nv, T, out, inp):
    """Several 256 x 256 tiles: ragged in every dimension (K ending on half a 32-wide step),
    the XCD-grouped tile order (4 x 8 tiles), and exactly one tile with one K step."""
    W, X = _case(T, out, inp, torch.bfloat16, seed=107 + inp)
    S = nv.global_scale(W, nv.GS_AMAX_448)
    r = nv.scale_search(W, None, S, nv.MSE, -3, 7, with_stats=False)
    _check(nv, X, W, S, r["packed"], r["scales"], what=f"{T}x{out}x{inp}")


def test_output_error_zero_residual_is_exactly_zero(nv):
    W, X = _case(256, 64, 128, torch.float32, seed=103)
    S = nv.global_scale(W, nv.GS_AMAX_448)
    r = nv.scale_search(W, None, S, nv.MSE, -3, 7, with_stats=False)
    W_hat = torch.from_numpy(oracle.dequant(r["packed"].cpu().numpy(), r["scales"].cpu().numpy(),
                                            float(S.item()))).to(DEV)
    err = nv.output_error(X, W_hat, r["packed"], r["scales"], S)
    torch.cuda.synchronize()
    assert (err.cpu().numpy() == 0).all()


def test_output_error_accumulates_chunks(nv):
    W, X = _case(512, 96, 256, torch.bfloat16, seed=105)
    S = nv.global_scale(W, nv.GS_AMAX_448)
    r = nv.scale_search(W, None, S, nv.MSE, 0, 0, with_stats=False)
    err = nv.output_error(X[:200], W, r["packed"], r["scales"], S)
    err = nv.output_error(X[200:], W, r["packed"], r["scales"], S, err=err, accumulate=True)
    torch.cuda.synchronize()
    o = oracle.output_error(host_w(X), host_w(W), r["packed"].cpu().numpy(),
                            r["scales"].cpu().numpy(), float(S.item()))
    np.testing.assert_allclose(err.cpu().numpy(), o, rtol=RTOL, atol=0)
    # no tokens: err unchanged when accumulating, zero otherwise
    before = err.clone()
    nv.output_error(X[:0], W, r["packed"], r["scales"], S, err=err, accumulate=True)
    torch.cuda.synchronize()
    assert torch.equal(err, before)
    z = nv.output_error(X[:0], W, r["packed"], r["scales"], S)
    torch.cuda.synchronize()
    assert (z.cpu().numpy() == 0).all()


def test_output_error_scale_rules_at_8b_attention_size(nv):
    """The 8B attention layer at full size (X 8192x4096, W 4096x4096), sampled rows against the
    oracle, and the ordering the pages report: Hessian-guided scales give a lower output error
    than max-abs scales."""
    cfg = workloads.CONFIGS["attn8b"]
    W = workloads.make_weights(cfg, DEV)
    sigma = workloads.make_sigma(cfg, DEV)
    X, _ = workloads.make_activation_chunk(cfg, sigma, 0, DEV)
    _, h = nv.diag_hessian(X)
    S = nv.global_scale(W, nv.GS_AMAX_256)
    rows = np.unique(np.concatenate([[0, 4095], np.random.default_rng(3).choice(4096, 40, replace=False)]))
    totals = {}
    for name, (hh, obj, lo, hi) in {"maxabs": (None, nv.MSE, 0, 0), "mse": (None, nv.MSE, -3, 7),
                                    "wmse": (h, nv.WMSE, -8, 7)}.items():
        r = nv.scale_search(W, hh, S, obj, lo, hi, with_stats=False)
        e, _ = _check(nv, X, W, S, r["packed"], r["scales"], rows=rows, what=name)
        totals[name] = float(e.sum())
    print(f"\n[attn8b] output error: {totals}; WMSE reduction vs max-abs "
          f"{1 - totals['wmse'] / totals['maxabs']:.3f}", flush=True)
    assert totals["wmse"] < totals["maxabs"]
