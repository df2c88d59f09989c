"""Shared helpers of the GPU parity tests: host copies in the oracle's formats, oracle and GPU
searches over [out, in] or [batch, out, in], and an element-by-element comparison."""
import numpy as np
import torch

import oracle


DEV = "cuda"


def host_w(W: torch.Tensor) -> np.ndarray:
    """W as the oracle takes it: float32, or bf16 bit patterns as uint16."""
    W = W.detach().cpu().contiguous()
    if W.dtype == torch.bfloat16:
        return W.view(torch.int16).numpy().view(np.uint16)
    return W.numpy().astype(np.float32)


OBJ = {"mse": oracle.MSE, "wmse": oracle.WMSE}


def oracle_search(W: torch.Tensor, h, S, objective, lo, hi, exhaustive):
    """Oracle over [out, in] or [batch, out, in]; h [in] / [batch, in] numpy; S list."""
    Wn = host_w(W)
    if Wn.ndim == 2:
        Wn, h, S = Wn[None], None if h is None else h[None], [S] if np.isscalar(S) else S
    res = [oracle.scale_search(Wn[b], None if h is None else h[b], OBJ[objective], lo, hi,
                               exhaustive, float(S[b])) for b in range(Wn.shape[0])]
    return {k: np.stack([r[k] for r in res]) for k in res[0]}


def gpu_search(nv, W, h, S, objective, lo, hi, exhaustive):
    r = nv.scale_search(W, h, S, nv.WMSE if objective == "wmse" else nv.MSE, lo, hi, exhaustive)
    torch.cuda.synchronize()
    out = {k: v.cpu().numpy() for k, v in r.items()}
    if W.dim() == 2:
        out = {k: v[None] for k, v in out.items()}
    return out


def assert_same(g, o, what=""):
    for k in ("scales", "offset", "loss", "packed"):
        a, b = g[k], o[k]
        if k == "loss":
            a, b = a.view(np.uint32), b.view(np.uint32)
        bad = np.argwhere(a != b)
        assert bad.size == 0, f"{what} {k}: {len(bad)} mismatches, first at {bad[:3].tolist()}"


