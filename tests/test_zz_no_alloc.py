"""The allocation-free activation entry point against the one that takes a workspace.

nvfp4_quantize_activations_noalloc is nvfp4_quantize_activations with the library's per-GPU
static scratch in place of the caller's workspace. Through the C ABI, on two calls in a row whose
second input is smaller (so the second call finds the first call's contents in the scratch),
every output must equal the workspace entry point's bit for bit: S, scale bytes and packed codes.
The pairs cover both internal paths (above 2^23 elements the global scale runs as its own two
kernels; below, the search reduces the amax partials itself), both element types and both
objectives.
"""
import numpy as np
import pytest
import torch

from gpu_helpers import DEV

pytestmark = pytest.mark.gpu


def _inputs(tokens, inp, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    sig = torch.exp(torch.randn(inp, generator=g, device=DEV) * 1.5)
    X = (torch.randn((tokens, inp), generator=g, device=DEV) * sig).to(dtype)
    h = torch.exp(torch.randn(inp, generator=g, device=DEV)).float()
    return X, h


def _outputs(tokens, inp):
    return (torch.full((1,), -1.0, device=DEV),
            torch.full((tokens * (inp // 16),), 255, dtype=torch.uint8, device=DEV),
            torch.full((tokens * (inp // 2),), 255, dtype=torch.uint8, device=DEV))


def _both(nv, X, h, objective, lo, hi, rule):
    T, n = X.shape
    S_a, sc_a, pk_a = _outputs(T, n)
    ws = torch.empty(nv.nvfp4_quantize_activations_workspace_size(T, n), dtype=torch.uint8,
                     device=DEV)
    hh = h if objective == nv.WMSE else None
    nv.nvfp4_quantize_activations(X, T, n, n, objective, hh, lo, hi, rule, S_a, sc_a, pk_a, ws)
    S_b, sc_b, pk_b = _outputs(T, n)
    nv.nvfp4_quantize_activations_noalloc(X, T, n, n, objective, hh, lo, hi, rule, S_b, sc_b,
                                          pk_b)
    torch.cuda.synchronize()
    return (S_a, sc_a, pk_a), (S_b, sc_b, pk_b)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("first,second", [((4096, 4096), (300, 512)),   # above, then below 2^23
                                          ((2048, 1024), (16, 2048)),   # below, then a decode batch
                                          ((8192, 2048), (4096, 2048))])  # above both times
def test_noalloc_matches_workspace_call(nv, dtype, first, second):
    for i, ((T, n), (objective, lo, hi, rule)) in enumerate(zip(
            (first, second), ((nv.MSE, -3, 7, nv.GS_AMAX_256), (nv.WMSE, -9, 6, nv.GS_AMAX_448)))):
        X, h = _inputs(T, n, dtype, seed=T + n + i)
        a, b = _both(nv, X, h, objective, lo, hi, rule)
        assert a[0].item() > 0 and a[0].item() == b[0].item(), f"S, call {i}"
        for name, x, y in (("scales", a[1], b[1]), ("packed", a[2], b[2])):
            bad = int((x != y).sum())
            assert bad == 0, f"{name}: {bad} bytes differ on call {i} ({T}x{n}, {dtype})"


def test_noalloc_without_S_out_and_repeated(nv):
    """No S output (the scratch's S slot serves), and the same call twice in a row."""
    X, h = _inputs(6000, 2048, torch.bfloat16, seed=3)
    T, n = X.shape
    ref = nv.quantize_activations(X, nv.MSE, -3, 7, nv.GS_AMAX_256)
    for _ in range(2):
        _, sc, pk = _outputs(T, n)
        nv.nvfp4_quantize_activations_noalloc(X, T, n, n, nv.MSE, None, -3, 7, nv.GS_AMAX_256,
                                              None, sc, pk)
        torch.cuda.synchronize()
        assert torch.equal(sc.reshape(ref["scales"].shape), ref["scales"])
        assert torch.equal(pk.reshape(ref["packed"].shape), ref["packed"])
