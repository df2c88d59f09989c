"""The library's calls captured in a HIP graph (through torch.cuda.graph): each replay gives the
bytes of the same calls made eagerly. The graph holds one layer's h and S (one
layer-statistics call) and its fused window + exhaustive search and nested MSE + WMSE search
(two search-rules calls); between replays the program clears the outputs and changes the
inputs eagerly and synchronises, and every replay is checked against a fresh eager run."""
import numpy as np
import pytest
import torch

from block_scale_search_amd import workloads
from gpu_helpers import DEV

pytestmark = pytest.mark.gpu


def _rules(nv, outs):
    specs = [(nv.WMSE, -9, 6, False), (nv.WMSE, 0, 0, True),      # fused launch
             (nv.MSE, -3, 7, False), (nv.WMSE, -8, 7, False)]     # nested launch
    return [dict(objective=o, lo=lo, hi=hi, exhaustive=e, **b)
            for (o, lo, hi, e), b in zip(specs, outs)]


def _buffers(o, n, n_rules):
    G = o * (n // 16)
    return [dict(scales=torch.empty(G, dtype=torch.uint8, device=DEV),
                 packed=torch.empty(G * 8, dtype=torch.uint8, device=DEV),
                 loss=torch.empty(G, dtype=torch.float32, device=DEV),
                 offset=torch.empty(G, dtype=torch.int8, device=DEV)) for _ in range(n_rules)]


def _issue(nv, X, W, st, stream):
    T, n = X.shape
    o = W.shape[0]
    nv.nvfp4_layer_statistics(X, T, n, n, st["h_acc"], st["h"], False, W, o, n,
                              nv.GS_AMAX_256, st["S"], st["ws"], stream=stream)
    rules = _rules(nv, st["outs"])
    nv.nvfp4_scale_search_rules(W, 1, o, n, n, o * n, 16, st["h"], n, st["S"], rules[:2],
                                stream=stream)
    nv.nvfp4_scale_search_rules(W, 1, o, n, n, o * n, 16, st["h"], n, st["S"], rules[2:],
                                stream=stream)


def _state(nv, T, n, o):
    return dict(h_acc=torch.empty(n, dtype=torch.float64, device=DEV),
                h=torch.empty(n, dtype=torch.float32, device=DEV),
                S=torch.empty(1, dtype=torch.float32, device=DEV),
                ws=torch.empty(max(16, nv.nvfp4_layer_statistics_workspace_size(T, n, o)),
                               dtype=torch.uint8, device=DEV),
                outs=_buffers(o, n, 4))


def _host(st):
    out = {"h_acc": st["h_acc"].cpu().numpy(), "h": st["h"].cpu().numpy(),
           "S": st["S"].cpu().numpy()}
    for i, b in enumerate(st["outs"]):
        for k, v in b.items():
            out[f"{i}.{k}"] = v.cpu().numpy()
    return out


def test_graph_replays_match_eager(nv):
    T, n, o = 1024, 1024, 96
    sigma = torch.exp(0.8 * torch.randn(n, generator=torch.Generator().manual_seed(3))).to(DEV)
    X = workloads.activations(T, sigma, seed=5, chunk_index=0, device=DEV)
    W = workloads.normal_weights(o, n, 0.02, 0.003, 25.0, seed=6, device=DEV)
    side = torch.cuda.Stream()
    graph_state, eager_state = _state(nv, T, n, o), _state(nv, T, n, o)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # eager warm-up on the capture stream
        _issue(nv, X, W, graph_state, side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        _issue(nv, X, W, graph_state, side)
    torch.cuda.synchronize()
    for rep in range(4):
        # the program's own eager work between replays: new inputs, cleared outputs
        if rep:
            X.copy_(workloads.activations(T, sigma, seed=5 + rep, chunk_index=0, device=DEV))
            W.copy_(workloads.normal_weights(o, n, 0.02, 0.003, 25.0, seed=6 + rep, device=DEV))
        for b in graph_state["outs"]:
            for v in b.values():
                v.zero_()
        graph_state["h"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _issue(nv, X, W, eager_state, torch.cuda.current_stream())
        torch.cuda.synchronize()
        got, want = _host(graph_state), _host(eager_state)
        for k in want:
            assert np.array_equal(got[k].view(np.uint8), want[k].view(np.uint8)), \
                f"replay {rep}: {k} differs from the eager call"
