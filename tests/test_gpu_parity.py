"""GPU parity: the HIP library (through the C ABI) against the CPU oracle, element by element.

Bar: scale bytes, packed codes and offsets bit-exact; losses bit-exact (same binary32 ops in the
same order); h within 1e-5 relative (in practice equal: both sum in binary64 and round once).
Sizes span several workgroups and ragged tails; the edge cases cover empty inputs, all-zero
groups, signed zeros, clipped windows at both ends of the code range, subnormal codes,
zero and wide-range h, and batched matrices.
"""
import numpy as np
import pytest
import torch

import oracle
from block_scale_search_amd import workloads

pytestmark = pytest.mark.gpu

H_RTOL = 1e-5


from gpu_helpers import DEV, assert_same, gpu_search, host_w, oracle_search


def _mat(out, inp, dtype, seed, outlier=0.003, batch=None):
    W = workloads.normal_weights(out, inp, 0.02, outlier, 25.0, seed, DEV, dtype, batch=batch)
    return W


def _h(inp, seed, batch=None, spread=2.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    shape = (inp,) if batch is None else (batch, inp)
    return torch.exp(torch.randn(shape, generator=g, device=DEV) * spread).float()


# ---------------------------------------------------------------------------------------------

def test_tiny_layer_all_modes(nv):
    """The tiny layer (W 256x256 fp32, X 512x256 bf16): h, S, every mode, bit-exact."""
    cfg = workloads.CONFIGS["tiny"]
    W = workloads.make_weights(cfg, DEV)
    sig = workloads.make_sigma(cfg, DEV)
    X, _ = workloads.make_activation_chunk(cfg, sig, 0, DEV)
    h_acc, h = nv.diag_hessian(X)
    acc_o, h_o = oracle.diag_hessian(host_w(X))
    np.testing.assert_allclose(h.cpu().numpy(), h_o, rtol=H_RTOL, atol=0)
    np.testing.assert_allclose(h_acc.cpu().numpy(), acc_o, rtol=1e-12, atol=0)
    S = nv.global_scale(W, nv.GS_AMAX_448)
    S_o = oracle.global_scale(host_w(W), oracle.GS_AMAX_448)
    assert S.item() == np.float32(S_o)
    hn = h.cpu().numpy()
    for mode in cfg.modes + [workloads.Mode("mse", exhaustive=True), workloads.Mode("wmse", -8, 7)]:
        g = gpu_search(nv, W, h if mode.objective == "wmse" else None, S, mode.objective,
                       mode.lo, mode.hi, mode.exhaustive)
        o = oracle_search(W, hn if mode.objective == "wmse" else None, S_o, mode.objective,
                          mode.lo, mode.hi, mode.exhaustive)
        assert_same(g, o, mode.label)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("shape", [(1, 37, 16), (1, 129, 48), (1, 300, 272), (3, 67, 160),
                                   (1, 5, 4096)])
def test_ragged_shapes(nv, dtype, shape):
    b, out, inp = shape
    W = _mat(out, inp, dtype, seed=out + inp, batch=None if b == 1 else b)
    h = _h(inp, seed=inp, batch=None if b == 1 else b)
    S = nv.global_scale(W, nv.GS_AMAX_256)
    Sn = S.cpu().numpy().reshape(-1)
    hn = h.cpu().numpy()
    for obj, lo, hi, exh in (("wmse", -9, 6, False), ("mse", -3, 7, False), ("wmse", -8, 7, False),
                             ("wmse", 0, 0, True)):
        g = gpu_search(nv, W, h if obj == "wmse" else None, S, obj, lo, hi, exh)
        o = oracle_search(W, hn if obj == "wmse" else None, Sn, obj, lo, hi, exh)
        assert_same(g, o, f"{shape} {obj} [{lo},{hi}] exh={exh}")


def test_padded_rows_and_strided_batch(nv):
    """ldw > in and a matrix stride larger than out * ldw: only the logical elements count."""
    base = _mat(40, 256, torch.bfloat16, seed=5, batch=2)
    big = torch.full((2, 48, 320), 7.0, dtype=torch.bfloat16, device=DEV)  # padding would win
    big[:, :40, :256] = base
    view = big[:, :40, :256]
    h = _h(256, seed=6, batch=2)
    S = nv.global_scale(view, nv.GS_AMAX_448)
    assert torch.equal(S, nv.global_scale(base.contiguous(), nv.GS_AMAX_448))
    for lo, hi, exh in ((-9, 6, False), (0, 0, True)):
        g = gpu_search(nv, view, h, S, "wmse", lo, hi, exh)
        o = oracle_search(base, h.cpu().numpy(), S.cpu().numpy(), "wmse", lo, hi, exh)
        assert_same(g, o, f"strided exh={exh}")


@pytest.mark.parametrize("window", [(-9, 6), (-3, 7), (0, 0), (-1, 0), (0, 5), (-125, 125),
                                    (-20, 3), (-2, 30)])
def test_windows(nv, window):
    lo, hi = window
    W = _mat(70, 512, torch.bfloat16, seed=11)
    h = _h(512, seed=12)
    S = nv.global_scale(W, nv.GS_AMAX_448)
    for obj in ("wmse", "mse"):
        g = gpu_search(nv, W, h if obj == "wmse" else None, S, obj, lo, hi, False)
        o = oracle_search(W, h.cpu().numpy() if obj == "wmse" else None, S.item(), obj, lo, hi,
                          False)
        assert_same(g, o, f"{obj} {window}")


def test_edge_groups(nv):
    """Zero groups, signed zeros, single non-zero, equal magnitudes, clipping at code 126,
    subnormal base codes, h zeros and extreme h."""
    out, inp = 64, 256
    W = _mat(out, inp, torch.float32, seed=21)
    W[0, :16] = 0.0
    W[1, :16] = -0.0
    W[2, :16] = 0.0
    W[2, 5] = -0.3
    W[3, :16] = 0.0125
    W[3, ::3] *= -1
    W[4, 16:32] = torch.linspace(-2.0, 2.0, 16, device=DEV)     # largest groups -> code 126
    W[5, :] *= 1e-4                                              # tiny groups -> low codes
    W[6, :] *= 3e-7                                              # subnormal base codes
    h = _h(inp, seed=22, spread=6.0)
    h[::7] = 0.0
    S = torch.tensor([2.0 / 448 / 6 * 0.7], device=DEV)         # top groups clip at 126
    for obj, lo, hi, exh in (("wmse", -9, 6, False), ("mse", -3, 7, False), ("wmse", 0, 0, True),
                             ("mse", 0, 0, True), ("wmse", -8, 7, False)):
        g = gpu_search(nv, W, h if obj == "wmse" else None, S, obj, lo, hi, exh)
        o = oracle_search(W, h.cpu().numpy() if obj == "wmse" else None, S.item(), obj, lo, hi,
                          exh)
        assert_same(g, o, f"edges {obj} [{lo},{hi}] exh={exh}")
    assert g["scales"][0, 0, 0] == 0 and g["scales"][0, 1, 0] == 0
    nib = oracle.unpack_nibbles(g["packed"][0])
    assert (nib[1, :16] == 8).all() and (nib[0, :16] == 0).all()
    base = gpu_search(nv, W, None, S, "mse", 0, 0, False)["scales"][0]
    assert base[4, 1] == 126 and base[6].max() == 1


def test_overflowing_losses_and_negative_h(nv):
    """Groups whose every candidate loss overflows to +inf keep their first candidate (the
    ascending scan never finds a strictly smaller loss), and a caller's h with negative entries
    (losses no longer sums of non-negative terms) still matches the oracle in every mode."""
    out, inp = 48, 256
    W = _mat(out, inp, torch.float32, seed=71)
    h = _h(inp, seed=72, spread=2.0)
    W[:16] *= 1e4
    hh = h.clone()
    hh[:64] = 3e38                                             # first 4 groups of rows 0..15 overflow
    hh[100:140] *= -1.0                                        # negative weights in other groups
    S = nv.global_scale(W, nv.GS_AMAX_448)
    for lo, hi, exh in ((-9, 6, False), (-8, 7, False), (0, 0, True), (-2, 1, False)):
        g = gpu_search(nv, W, hh, S, "wmse", lo, hi, exh)
        o = oracle_search(W, hh.cpu().numpy(), S.item(), "wmse", lo, hi, exh)
        assert_same(g, o, f"overflow/negative h [{lo},{hi}] exh={exh}")
    assert np.isinf(g["loss"][0, :16, :4]).all()


def test_tiny_global_scale_subnormal_codes(nv):
    """A global scale so small that the lowest codes' effective scales are subnormal binary32
    values (their reciprocals still finite), with h large enough that losses do not flush."""
    W = _mat(32, 128, torch.float32, seed=31) * 1e-33
    h = _h(128, seed=32) * 1e30
    S = torch.tensor([float(np.float32(2.6e-36))], device=DEV)
    eff, _ = oracle.scale_tables(S.item())
    assert eff[1] < np.finfo(np.float32).tiny            # subnormal effective scale
    for obj, lo, hi, exh in (("wmse", -9, 6, False), ("wmse", 0, 0, True), ("mse", 0, 0, True)):
        g = gpu_search(nv, W, h if obj == "wmse" else None, S, obj, lo, hi, exh)
        o = oracle_search(W, h.cpu().numpy() if obj == "wmse" else None, S.item(), obj, lo, hi,
                          exh)
        assert_same(g, o, f"tiny S {obj} exh={exh}")


@pytest.mark.parametrize("s_scale", [1.0, 1e-3, 30.0])
def test_exhaustive_pruning_boundaries(nv, s_scale):
    """Exhaustive mode against the oracle where its exact prunings bite differently per lane:
    groups whose largest weight has h = 0 (no lower bound, deep contractions can win), huge h at
    the largest weight (early stop), all-small groups (constant top region reached early),
    and global scales that move the top region towards either end of the code range."""
    out, inp = 96, 256
    W = _mat(out, inp, torch.float32, seed=61)
    g = torch.Generator(device=DEV)
    g.manual_seed(62)
    h = torch.exp(torch.randn(inp, generator=g, device=DEV) * 3.0)
    Wg = W.view(out, inp // 16, 16)
    imax = Wg.abs().argmax(-1)                               # column of each group's max
    cols = (torch.arange(inp // 16, device=DEV) * 16)[None, :] + imax
    hz = h.clone()
    hz[cols[::3].reshape(-1)] = 0.0                          # every third row: h = 0 at the max
    hz[cols[1::3].reshape(-1)] *= 1e6                        # next: h huge at the max
    W[2::3] *= 1e-3                                          # last: tiny groups
    S = nv.global_scale(W, nv.GS_AMAX_448) * s_scale
    for obj, hh in (("wmse", hz), ("mse", None)):
        gg = gpu_search(nv, W, hh, S, obj, 0, 0, True)
        o = oracle_search(W, None if hh is None else hh.cpu().numpy(), S.item(), obj, 0, 0, True)
        assert_same(gg, o, f"exhaustive {obj} S x{s_scale}")


def test_pack_parity_and_window_zero(nv):
    W = _mat(96, 384, torch.bfloat16, seed=41)
    S = nv.global_scale(W, nv.GS_AMAX_448)
    g = torch.Generator(device=DEV)
    g.manual_seed(42)
    scales = torch.randint(0, 127, (96, 24), generator=g, device=DEV, dtype=torch.int32).to(torch.uint8)
    p = nv.pack(W, scales, S)
    po = oracle.pack(host_w(W), scales.cpu().numpy(), S.item())
    np.testing.assert_array_equal(p.cpu().numpy(), po)
    r = nv.scale_search(W, None, S, nv.MSE, 0, 0)
    np.testing.assert_array_equal(nv.pack(W, r["scales"], S).cpu().numpy(),
                                  r["packed"].cpu().numpy())


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_pack_strided_batched_ragged(nv, dtype):
    """Pack at given scales on padded rows (ldw > in), a batch of matrices with a gap between
    them, a group count per row that is not a multiple of the 64 groups a wave covers, and
    scale bytes over the whole 0..126 range, against the oracle matrix by matrix."""
    B, out, inp, ldw = 3, 37, 208, 232
    base = _mat(B * 40, ldw, dtype, seed=81).reshape(B, 40, ldw)
    W = base[:, :out, :inp]                                     # strided view, gap between matrices
    S = nv.global_scale(W, nv.GS_AMAX_448)
    g = torch.Generator(device=DEV)
    g.manual_seed(82)
    scales = torch.randint(0, 127, (B, out, inp // 16), generator=g, device=DEV,
                           dtype=torch.int32).to(torch.uint8)
    scales[:, 0, :] = torch.arange(inp // 16, device=DEV, dtype=torch.uint8) * 9  # 0, 9, .., 117
    p = nv.pack(W, scales, S).cpu().numpy()
    for b in range(B):
        po = oracle.pack(host_w(W[b]), scales[b].cpu().numpy(), float(S[b].item()))
        np.testing.assert_array_equal(p[b], po, err_msg=f"matrix {b}")


def test_repeatable(nv):
    W = _mat(512, 1024, torch.bfloat16, seed=51)
    h = _h(1024, seed=52)
    S = nv.global_scale(W, nv.GS_AMAX_448)
    a = nv.scale_search(W, h, S, nv.WMSE, -9, 6)
    b = nv.scale_search(W, h, S, nv.WMSE, -9, 6)
    for k in a:
        assert torch.equal(a[k], b[k])
    X = workloads.activations(1000, torch.ones(1024, device=DEV), seed=53, device=DEV)
    h1 = nv.diag_hessian(X)[0]
    h2 = nv.diag_hessian(X)[0]
    assert torch.equal(h1, h2)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T,inp", [(1, 8), (127, 24), (511, 512), (512, 136), (513, 1000),
                                   (3000, 4096), (5000, 200)])
def test_hessian(nv, dtype, T, inp):
    sig = workloads.channel_sigma(inp, 1.5, seed=inp, device=DEV)
    X = workloads.activations(T, sig, seed=T, device=DEV, dtype=dtype)
    acc, h = nv.diag_hessian(X)
    acc_o, h_o = oracle.diag_hessian(host_w(X))
    np.testing.assert_allclose(acc.cpu().numpy(), acc_o, rtol=1e-12, atol=0)
    np.testing.assert_allclose(h.cpu().numpy(), h_o, rtol=H_RTOL, atol=0)


def test_hessian_padded_and_chunked(nv):
    full = workloads.activations(2500, torch.ones(640, device=DEV), seed=61, device=DEV)
    big = torch.zeros((2500, 704), dtype=torch.bfloat16, device=DEV)
    big[:, :640] = full
    X = big[:, :640]
    acc = None
    acc_o = None
    for t0 in range(0, 2500, 700):
        acc, h = nv.diag_hessian(X[t0:t0 + 700], acc, accumulate=acc is not None)
        acc_o, h_o = oracle.diag_hessian(host_w(full[t0:t0 + 700]), acc_o)
    np.testing.assert_allclose(acc.cpu().numpy(), acc_o, rtol=1e-12, atol=0)
    np.testing.assert_allclose(h.cpu().numpy(), h_o, rtol=H_RTOL, atol=0)
    # empty token chunk keeps / clears the accumulator
    acc2, h2 = nv.diag_hessian(X[:0], acc.clone(), accumulate=True)
    assert torch.equal(acc2, acc)
    acc3, h3 = nv.diag_hessian(X[:0], acc.clone(), accumulate=False)
    assert (acc3 == 0).all() and (h3 == 0).all()


def test_hessian_batched_segments(nv):
    counts = np.array([300, 0, 1, 129, 1000, 0, 77, 128], dtype=np.int64)
    offs = np.concatenate([[0], np.cumsum(counts)])
    T, inp = int(offs[-1]), 264
    sig = workloads.channel_sigma(inp, 1.0, seed=71, device=DEV)
    X = workloads.activations(T, sig, seed=72, device=DEV)
    seg = torch.from_numpy(offs).to(DEV)
    acc, h = nv.diag_hessian_batched(X, seg)
    Xn = host_w(X)
    for e in range(len(counts)):
        a_o, h_o = oracle.diag_hessian(Xn[offs[e]:offs[e + 1]])
        np.testing.assert_allclose(acc[e].cpu().numpy(), a_o, rtol=1e-12, atol=0)
        np.testing.assert_allclose(h[e].cpu().numpy(), h_o, rtol=H_RTOL, atol=0)
    acc2, _ = nv.diag_hessian_batched(X, seg, acc.clone(), accumulate=True)
    np.testing.assert_allclose(acc2.cpu().numpy(), 2 * acc.cpu().numpy(), rtol=1e-12)


def test_workspace_reuse(nv):
    """One workspace serves a sequence of calls (token counts and element types vary) with no
    clearing in between: nothing a call leaves behind changes the next result."""
    n = 520
    ws = torch.full((nv.nvfp4_diag_hessian_workspace_size(5000, n, 1),), 0xA5, dtype=torch.uint8,
                     device=DEV)
    for T, dt in ((3000, torch.bfloat16), (100, torch.float32), (5000, torch.bfloat16),
                  (0, torch.bfloat16), (513, torch.float32), (3000, torch.bfloat16)):
        X = workloads.activations(T, torch.ones(n, device=DEV), seed=T + 1, device=DEV, dtype=dt)
        acc = torch.empty(n, dtype=torch.float64, device=DEV)
        h = torch.empty(n, dtype=torch.float32, device=DEV)
        nv.nvfp4_diag_hessian(X, T, n, n, acc, h, False, ws)
        want = oracle.diag_hessian(host_w(X))[0] if T else np.zeros(n)
        np.testing.assert_allclose(acc.cpu().numpy(), want, rtol=1e-12)
    offs = torch.tensor([0, 10, 10, 600, 1700], dtype=torch.int64, device=DEV)
    wsb = torch.full((nv.nvfp4_diag_hessian_workspace_size(1700, n, 4),), 0xA5, dtype=torch.uint8,
                      device=DEV)
    for rep in range(3):
        X = workloads.activations(1700, torch.ones(n, device=DEV), seed=rep, device=DEV)
        acc = torch.empty(4 * n, dtype=torch.float64, device=DEV)
        nv.nvfp4_diag_hessian_batched(X, offs, 4, 1700, n, n, acc, None, False, wsb)
        Xn = host_w(X)
        for e in range(4):
            o0, o1 = int(offs[e]), int(offs[e + 1])
            want = oracle.diag_hessian(Xn[o0:o1])[0] if o1 > o0 else np.zeros(n)
            np.testing.assert_allclose(acc[e * n:(e + 1) * n].cpu().numpy(), want, rtol=1e-12)
    wss = torch.zeros((nv.nvfp4_global_scale_workspace_size(1, 4096, 4096),), dtype=torch.uint8,
                      device=DEV)
    for out, inp, dt in ((512, 4096, torch.bfloat16), (64, 512, torch.float32), (4096, 4096, torch.bfloat16)):
        W = _mat(out, inp, dt, seed=out + inp)
        S = torch.empty(1, dtype=torch.float32, device=DEV)
        nv.nvfp4_global_scale(W, 1, out, inp, inp, out * inp, nv.GS_AMAX_448, S, wss)
        assert S.item() == np.float32(oracle.global_scale(host_w(W), oracle.GS_AMAX_448))


def test_global_scale_many_calls(nv):
    """Many back-to-back global-scale calls (1-4 matrices, both element types) on one reused
    workspace, against the oracle each time."""
    ws = torch.zeros(nv.nvfp4_global_scale_workspace_size(4, 64 + 17 * 60, 512), dtype=torch.uint8,
                     device=DEV)
    mats, outs = [], []
    for i in range(60):
        b = 1 + i % 4
        W = _mat(64 + 17 * i, 512, torch.bfloat16 if i % 2 else torch.float32, seed=900 + i,
                 batch=None if b == 1 else b)
        bb, o, n = (1,) + tuple(W.shape) if W.dim() == 2 else tuple(W.shape)
        S = torch.empty(bb, dtype=torch.float32, device=DEV)
        nv.nvfp4_global_scale(W, bb, o, n, n, o * n, nv.GS_AMAX_256, S, ws)
        mats.append(W)
        outs.append(S)
    torch.cuda.synchronize()
    for W, S in zip(mats, outs):
        Wb = W if W.dim() == 3 else W[None]
        for b in range(Wb.shape[0]):
            assert S[b].item() == np.float32(oracle.global_scale(host_w(Wb[b]), oracle.GS_AMAX_256))


def test_global_scale_rules_and_batch(nv):
    W = _mat(33, 96, torch.bfloat16, seed=81, batch=5)
    W[3] = 0
    for rule, orule in ((nv.GS_AMAX_448, oracle.GS_AMAX_448), (nv.GS_AMAX_256, oracle.GS_AMAX_256)):
        S = nv.global_scale(W, rule).cpu().numpy()
        for b in range(5):
            assert S[b] == np.float32(oracle.global_scale(host_w(W[b]), orule))
    assert S[3] == 1.0


def test_empty_inputs(nv):
    W = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    S = nv.global_scale(W)
    assert S.item() == 1.0
    r = nv.scale_search(W, torch.ones(64, device=DEV), S, nv.WMSE)
    assert r["scales"].numel() == 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_hessian_deferred_chunks(nv, dtype):
    """Deferred mode: chunks only add row-group sums into the workspace (a shorter last
    chunk included), one finalize at the end; equal to the oracle over all tokens, and a
    second finalize with accumulate adds the same sums again."""
    g = torch.Generator(device=DEV)
    g.manual_seed(77)
    inp = 1040
    sizes = [3000, 3000, 3000, 1234]
    chunks = [(torch.randn((t, inp), generator=g, device=DEV) *
               torch.exp(torch.randn(inp, generator=g, device=DEV))).to(dtype) for t in sizes]
    T0 = sizes[0]
    ws = torch.empty(nv.nvfp4_diag_hessian_workspace_size(T0, inp, 1), dtype=torch.uint8, device=DEV)
    for i, X in enumerate(chunks):
        nv.nvfp4_diag_hessian(X, X.shape[0], inp, inp, None, None, i > 0, ws)
    h_acc = torch.empty(inp, dtype=torch.float64, device=DEV)
    h = torch.empty(inp, dtype=torch.float32, device=DEV)
    nv.nvfp4_diag_hessian_finalize(dtype, T0, inp, h_acc, h, False, ws)
    torch.cuda.synchronize()
    acc_o, h_o = oracle.diag_hessian(host_w(torch.cat(chunks)))
    np.testing.assert_allclose(h_acc.cpu().numpy(), acc_o, rtol=1e-12, atol=0)
    np.testing.assert_allclose(h.cpu().numpy(), h_o, rtol=H_RTOL, atol=0)
    nv.nvfp4_diag_hessian_finalize(dtype, T0, inp, h_acc, None, True, ws)
    torch.cuda.synchronize()
    np.testing.assert_allclose(h_acc.cpu().numpy(), 2 * acc_o, rtol=1e-12, atol=0)


@pytest.mark.parametrize("inp,sizes,ws_tokens", [
    (4096, [1025, 1024], 8192),               # workspace larger than the first chunk needs
    (4096, [7936, 7680, 1025, 17, 1], 7936),
    (1040, [3000, 16, 3000, 1], 3000),
])
def test_hessian_deferred_ragged_chunks(nv, inp, sizes, ws_tokens):
    """Deferred mode with chunks of falling and ragged sizes (the first the longest), some
    with fewer row-group slots than the first: every token lands in a slot the first chunk
    initialised, so the finalize over the first chunk's layout equals the oracle over all
    tokens."""
    g = torch.Generator(device=DEV)
    g.manual_seed(sum(sizes) + inp)
    chunks = [(torch.randn((t, inp), generator=g, device=DEV) *
               torch.exp(torch.randn(inp, generator=g, device=DEV))).to(torch.bfloat16)
              for t in sizes]
    ws = torch.empty(nv.nvfp4_diag_hessian_workspace_size(ws_tokens, inp, 1), dtype=torch.uint8,
                     device=DEV)
    for i, X in enumerate(chunks):
        nv.nvfp4_diag_hessian(X, X.shape[0], inp, inp, None, None, i > 0, ws)
    h_acc = torch.empty(inp, dtype=torch.float64, device=DEV)
    h = torch.empty(inp, dtype=torch.float32, device=DEV)
    nv.nvfp4_diag_hessian_finalize(torch.bfloat16, sizes[0], inp, h_acc, h, False, ws)
    torch.cuda.synchronize()
    acc_o, h_o = oracle.diag_hessian(host_w(torch.cat(chunks)))
    np.testing.assert_allclose(h_acc.cpu().numpy(), acc_o, rtol=1e-12, atol=0)
    np.testing.assert_allclose(h.cpu().numpy(), h_o, rtol=H_RTOL, atol=0)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("inp,sizes,ldx", [
    (4096, [8192] * 8, 4096),                   # the 70B-shaped calibration set's chunk shape
    (1040, [3000, 0, 17, 1234, 1], 1040),       # ragged sizes, an empty chunk
    (640, [2500, 700], 704),                     # padded rows
    (24, [1], 24),                               # one chunk of one token
    (512, [37 * (i % 5) + 1 for i in range(64)], 512),   # the largest chunk count, 64
])
def test_hessian_chunks_one_launch(nv, dtype, inp, sizes, ldx):
    """Chunks at separate addresses in one partial launch and one finalize: h over all their
    tokens against the oracle (binary64 sums within 1e-12, h within 1e-5), and accumulate
    continues from h_acc."""
    g = torch.Generator(device=DEV)
    g.manual_seed(sum(sizes) + inp + ldx)
    sig = torch.exp(torch.randn(inp, generator=g, device=DEV) * 1.5)
    full = [(torch.randn((t, ldx), generator=g, device=DEV) *
             torch.nn.functional.pad(sig, (0, ldx - inp), value=1.0)).to(dtype) for t in sizes]
    chunks = [f[:, :inp] for f in full]
    ws = torch.empty(max(16, nv.nvfp4_diag_hessian_chunks_workspace_size(sizes, inp)),
                     dtype=torch.uint8, device=DEV)
    h_acc = torch.empty(inp, dtype=torch.float64, device=DEV)
    h = torch.empty(inp, dtype=torch.float32, device=DEV)
    nv.nvfp4_diag_hessian_chunks(chunks, inp, ldx, h_acc, h, False, ws)
    torch.cuda.synchronize()
    acc_o, h_o = oracle.diag_hessian(host_w(torch.cat(chunks)))
    np.testing.assert_allclose(h_acc.cpu().numpy(), acc_o, rtol=1e-12, atol=0)
    np.testing.assert_allclose(h.cpu().numpy(), h_o, rtol=H_RTOL, atol=0)
    nv.nvfp4_diag_hessian_chunks(chunks, inp, ldx, h_acc, None, True, ws)
    torch.cuda.synchronize()
    np.testing.assert_allclose(h_acc.cpu().numpy(), 2 * acc_o, rtol=1e-12, atol=0)
