"""Thin Python binding of the C ABI in ``include/nvfp4.h`` (ctypes over ``libnvfp4.so``).

Each ``nvfp4_*`` function here has the name and arguments of the C entry point, with torch
tensors in place of device pointers; it only checks that tensors live on the GPU with the
expected dtype, contiguity and size, passes their pointers and the current torch stream, and
raises ``Nvfp4Error`` on a non-OK status. Every computation runs in the library's HIP kernels;
there is no CPU path. Importing this module fails if the library has not been built
(``python -m block_scale_search_amd.build``).

The convenience wrappers at the end (``diag_hessian``, ``layer_statistics``, ``global_scale``,
``scale_search``, ``scale_search_rules``, ``scale_search_proposal``, ``pack``, ``quantize_activations``, ``gptq``,
``output_error``) allocate outputs and workspaces with torch and call the entry points.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m block_scale_search_amd.build`")
_lib = ctypes.CDLL(_LIB_PATH)

OK, ERR_NULL, ERR_SHAPE, ERR_DTYPE, ERR_ALIGN, ERR_WINDOW, ERR_ARG, ERR_WORKSPACE, ERR_HIP = range(9)
DTYPE_F32, DTYPE_BF16 = 0, 1
MSE, WMSE = 0, 1
GS_AMAX_448, GS_AMAX_256 = 0, 1

_P, _I64, _I32, _I, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int, ctypes.c_size_t

class SearchRule(ctypes.Structure):
    """``nvfp4_search_rule``: one objective and window with its output pointers."""
    _fields_ = [("objective", ctypes.c_int32), ("lo", ctypes.c_int32), ("hi", ctypes.c_int32),
                ("exhaustive", ctypes.c_int32), ("scales", ctypes.c_void_p),
                ("packed", ctypes.c_void_p), ("loss", ctypes.c_void_p),
                ("offset", ctypes.c_void_p)]


_SIGS = {
    "nvfp4_status_string": ([_I], ctypes.c_char_p),
    "nvfp4_version": ([], ctypes.c_char_p),
    "nvfp4_diag_hessian_workspace_size": ([_I64, _I64, _I64], _SZ),
    "nvfp4_diag_hessian": ([_P, _I, _I64, _I64, _I64, _P, _P, _I, _P, _SZ, _P], _I),
    "nvfp4_diag_hessian_finalize": ([_I, _I64, _I64, _P, _P, _I, _P, _SZ, _P], _I),
    "nvfp4_diag_hessian_batched": ([_P, _I, _P, _I64, _I64, _I64, _I64, _P, _P, _I, _P, _SZ, _P], _I),
    "nvfp4_diag_hessian_chunks_workspace_size": ([_P, _I64, _I64], _SZ),
    "nvfp4_diag_hessian_chunks": ([_P, _I, _P, _I64, _I64, _I64, _P, _P, _I, _P, _SZ, _P], _I),
    "nvfp4_global_scale_workspace_size": ([_I64, _I64, _I64], _SZ),
    "nvfp4_global_scale": ([_P, _I, _I64, _I64, _I64, _I64, _I64, _I, _P, _P, _SZ, _P], _I),
    "nvfp4_layer_statistics_workspace_size": ([_I64, _I64, _I64], _SZ),
    "nvfp4_layer_statistics": ([_P, _I, _I64, _I64, _I64, _P, _P, _I, _P, _I, _I64, _I64, _I, _P,
                                _P, _SZ, _P], _I),
    "nvfp4_scale_search": ([_P, _I, _I64, _I64, _I64, _I64, _I64, _I32, _P, _I64, _I, _I32, _I32, _I,
                            _P, _P, _P, _P, _P, _P], _I),
    "nvfp4_scale_search_rules": ([_P, _I, _I64, _I64, _I64, _I64, _I64, _I32, _P, _I64, _P,
                                  ctypes.POINTER(SearchRule), _I32, _P], _I),
    "nvfp4_scale_search_scored": ([_P, _I, _I64, _I64, _I64, _I64, _I64, _I32, _P, _I64, _I, _I32,
                                   _P, _P, _P], _I),
    "nvfp4_scale_search_proposal": ([_P, _I, _I64, _I64, _I64, _I64, _I64, _I32, _P, _I64, _I,
                                     _I32, _I32, _P, _P, _P, _P, _P, _P, _P, _P], _I),
    "nvfp4_pack": ([_P, _I, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P], _I),
    "nvfp4_quantize_activations_workspace_size": ([_I64, _I64], _SZ),
    "nvfp4_quantize_activations": ([_P, _I, _I64, _I64, _I64, _I, _P, _I32, _I32, _I, _P, _P, _P,
                                    _P, _SZ, _P], _I),
    "nvfp4_quantize_activations_noalloc": ([_P, _I, _I64, _I64, _I64, _I, _P, _I32, _I32, _I,
                                            _P, _P, _P, _P], _I),
    "nvfp4_gptq_workspace_size": ([_I64, _I64], _SZ),
    "nvfp4_gptq": ([_P, _I, _I64, _I64, _I64, _P, _P, _I, _I32, _I32, _P, _P, _P, _P, _P, _SZ,
                    _P], _I),
    "nvfp4_output_error_workspace_size": ([_I64, _I64, _I64], _SZ),
    "nvfp4_output_error": ([_P, _I, _I64, _I64, _I64, _P, _I, _I64, _I64, _P, _P, _P, _P, _I,
                            _P, _SZ, _P], _I),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTS = tuple(_SIGS)


class Nvfp4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.nvfp4_status_string(status).decode()}")


def _check(status: int, where: str) -> None:
    if status != OK:
        raise Nvfp4Error(status, where)


def _run(fname: str, args: tuple, prepare: bool):
    """Call C entry point `fname` with marshalled `args`, or (prepare=True) return a
    zero-argument callable that makes exactly that call; the tensors behind the pointers must
    then stay alive and unchanged in size while the callable is used."""
    f = getattr(_lib, fname)
    if not prepare:
        _check(f(*args), fname)
        return None

    def call():
        _check(f(*args), fname)
    return call


def _dev(t: torch.Tensor | None, name: str, dtypes=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a tensor on the GPU")
    if dtypes is not None and t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    return ctypes.c_void_p(t.data_ptr())


def _wdtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported element type {t.dtype} (float32 or bfloat16)")


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, numel: int, name: str):
    if not t.is_contiguous() or t.numel() < numel:
        raise ValueError(f"{name} must be contiguous with at least {numel} elements")


def nvfp4_version() -> str:
    return _lib.nvfp4_version().decode()


def nvfp4_status_string(status: int) -> str:
    return _lib.nvfp4_status_string(status).decode()


def nvfp4_diag_hessian_workspace_size(tokens: int, inp: int, segments: int = 1) -> int:
    return int(_lib.nvfp4_diag_hessian_workspace_size(tokens, inp, segments))


def _i64_array(values):
    return (ctypes.c_int64 * len(values))(*[int(v) for v in values])


def nvfp4_diag_hessian_chunks_workspace_size(tokens, inp: int) -> int:
    t = _i64_array(tokens)
    return int(_lib.nvfp4_diag_hessian_chunks_workspace_size(t, len(tokens), inp))


def nvfp4_diag_hessian_chunks(X_chunks, inp, ldx, h_acc, h, accumulate, workspace, stream=None,
                              prepare=False):
    """h over several token chunks (tensors [tokens_c, in] at separate addresses) in one partial
    launch and one finalize."""
    if not X_chunks:
        raise ValueError("at least one chunk")
    dt = {_wdtype(X) for X in X_chunks}
    if len(dt) != 1:
        raise TypeError("every chunk must have the same element type")
    _need(h_acc, inp, "h_acc")
    if h is not None:
        _need(h, inp, "h")
    ptrs = (ctypes.c_void_p * len(X_chunks))(*[_dev(X, "X").value for X in X_chunks])
    toks = _i64_array([X.shape[0] for X in X_chunks])
    args = (ptrs, dt.pop(), toks, len(X_chunks), inp, ldx, _dev(h_acc, "h_acc", (torch.float64,)),
            _dev(h, "h", (torch.float32,)), int(accumulate), _dev(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream))
    return _run("nvfp4_diag_hessian_chunks", args, prepare)


def nvfp4_global_scale_workspace_size(batch: int, out: int, inp: int) -> int:
    return int(_lib.nvfp4_global_scale_workspace_size(batch, out, inp))


def nvfp4_layer_statistics_workspace_size(tokens: int, inp: int, out: int) -> int:
    return int(_lib.nvfp4_layer_statistics_workspace_size(tokens, inp, out))


def nvfp4_diag_hessian(X, tokens, inp, ldx, h_acc, h, accumulate, workspace, stream=None, prepare=False):
    """h_acc = h = None: deferred mode (row-group sums into the workspace only)."""
    if h_acc is not None:
        _need(h_acc, inp, "h_acc")
    if h is not None:
        _need(h, inp, "h")
    return _run("nvfp4_diag_hessian", (
        _dev(X, "X", (torch.float32, torch.bfloat16)), _wdtype(X), tokens, inp, ldx,
        _dev(h_acc, "h_acc", (torch.float64,)), _dev(h, "h", (torch.float32,)), int(accumulate),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)), prepare)


def nvfp4_diag_hessian_finalize(X_dtype, tokens, inp, h_acc, h, accumulate, workspace,
                                stream=None, prepare=False):
    """Finalize of deferred nvfp4_diag_hessian calls (X_dtype: torch.bfloat16 or float32)."""
    dt = DTYPE_BF16 if X_dtype == torch.bfloat16 else DTYPE_F32
    return _run("nvfp4_diag_hessian_finalize", (
        dt, tokens, inp, _dev(h_acc, "h_acc", (torch.float64,)), _dev(h, "h", (torch.float32,)),
        int(accumulate), _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)), prepare)


def nvfp4_diag_hessian_batched(X, seg_offsets, segments, total_tokens, inp, ldx, h_acc, h,
                               accumulate, workspace, stream=None, prepare=False):
    _need(h_acc, segments * inp, "h_acc")
    if h is not None:
        _need(h, segments * inp, "h")
    return _run("nvfp4_diag_hessian_batched", (
        _dev(X, "X", (torch.float32, torch.bfloat16)), _wdtype(X),
        _dev(seg_offsets, "seg_offsets", (torch.int64,)), segments, total_tokens, inp, ldx,
        _dev(h_acc, "h_acc", (torch.float64,)), _dev(h, "h", (torch.float32,)), int(accumulate),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)), prepare)


def nvfp4_global_scale(W, batch, out, inp, ldw, stride_w, rule, S, workspace, stream=None, prepare=False):
    _need(S, batch, "S")
    return _run("nvfp4_global_scale", (
        _dev(W, "W", (torch.float32, torch.bfloat16)), _wdtype(W), batch, out, inp, ldw, stride_w,
        rule, _dev(S, "S", (torch.float32,)), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)), prepare)


def nvfp4_layer_statistics(X, tokens, inp, ldx, h_acc, h, accumulate, W, out, ldw, rule, S,
                           workspace, stream=None, prepare=False):
    _need(h_acc, inp, "h_acc")
    if h is not None:
        _need(h, inp, "h")
    _need(S, 1, "S")
    return _run("nvfp4_layer_statistics", (
        _dev(X, "X", (torch.float32, torch.bfloat16)), _wdtype(X), tokens, inp, ldx,
        _dev(h_acc, "h_acc", (torch.float64,)), _dev(h, "h", (torch.float32,)), int(accumulate),
        _dev(W, "W", (torch.float32, torch.bfloat16)), _wdtype(W), out, ldw, rule,
        _dev(S, "S", (torch.float32,)), _dev(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(stream)), prepare)


def nvfp4_scale_search(W, batch, out, inp, ldw, stride_w, group_size, h, stride_h, objective,
                       lo, hi, exhaustive, S, scales, packed, loss=None, offset=None, stream=None, prepare=False):
    G = batch * out * (inp // 16)
    _need(scales, G, "scales")
    _need(packed, G * 8, "packed")
    _need(S, batch, "S")
    if loss is not None:
        _need(loss, G, "loss")
    if offset is not None:
        _need(offset, G, "offset")
    return _run("nvfp4_scale_search", (
        _dev(W, "W", (torch.float32, torch.bfloat16)), _wdtype(W), batch, out, inp, ldw, stride_w,
        group_size, _dev(h, "h", (torch.float32,)), stride_h, objective, lo, hi, int(exhaustive),
        _dev(S, "S", (torch.float32,)), _dev(scales, "scales", (torch.uint8,)),
        _dev(packed, "packed", (torch.uint8,)), _dev(loss, "loss", (torch.float32,)),
        _dev(offset, "offset", (torch.int8,)), _stream(stream)), prepare)


def nvfp4_scale_search_rules(W, batch, out, inp, ldw, stride_w, group_size, h, stride_h, S, rules,
                             stream=None, prepare=False):
    """rules: sequence of dicts with keys objective, lo, hi, exhaustive, scales, packed and
    optionally loss, offset (tensors)."""
    G = batch * out * (inp // 16)
    _need(S, batch, "S")
    arr = (SearchRule * len(rules))()
    for k, r in enumerate(rules):
        _need(r["scales"], G, "scales")
        _need(r["packed"], G * 8, "packed")
        loss, offset = r.get("loss"), r.get("offset")
        if loss is not None:
            _need(loss, G, "loss")
        if offset is not None:
            _need(offset, G, "offset")
        p = lambda t, name, dt: None if t is None else _dev(t, name, dt).value
        arr[k] = SearchRule(int(r["objective"]), int(r["lo"]), int(r["hi"]), int(r["exhaustive"]),
                            p(r["scales"], "scales", (torch.uint8,)),
                            p(r["packed"], "packed", (torch.uint8,)),
                            p(loss, "loss", (torch.float32,)), p(offset, "offset", (torch.int8,)))
    call = _run("nvfp4_scale_search_rules", (
        _dev(W, "W", (torch.float32, torch.bfloat16)), _wdtype(W), batch, out, inp, ldw, stride_w,
        group_size, _dev(h, "h", (torch.float32,)), stride_h, _dev(S, "S", (torch.float32,)),
        arr, len(rules), _stream(stream)), prepare)
    if prepare:
        return lambda: (arr, call())[1]     # the closure keeps the rule array alive
    return None


def nvfp4_scale_search_scored(W, batch, out, inp, ldw, stride_w, group_size, h, stride_h,
                              objective, centre_lo, S, count, stream=None, prepare=False):
    _need(S, batch, "S")
    _need(count, 1, "count")
    return _run("nvfp4_scale_search_scored", (
        _dev(W, "W", (torch.float32, torch.bfloat16)), _wdtype(W), batch, out, inp, ldw, stride_w,
        group_size, _dev(h, "h", (torch.float32,)), stride_h, objective, centre_lo,
        _dev(S, "S", (torch.float32,)), _dev(count, "count", (torch.int64,)), _stream(stream)),
        prepare)


def nvfp4_scale_search_proposal(W, batch, out, inp, ldw, stride_w, group_size, h, stride_h,
                                objective, lo, hi, center, incoming, S, scales, packed, loss=None,
                                offset=None, stream=None, prepare=False):
    G = batch * out * (inp // 16)
    _need(scales, G, "scales")
    _need(packed, G * 8, "packed")
    _need(center, G, "center")
    if incoming is not None:
        _need(incoming, G, "incoming")
    _need(S, batch, "S")
    if loss is not None:
        _need(loss, G, "loss")
    if offset is not None:
        _need(offset, G, "offset")
    return _run("nvfp4_scale_search_proposal", (
        _dev(W, "W", (torch.float32, torch.bfloat16)), _wdtype(W), batch, out, inp, ldw, stride_w,
        group_size, _dev(h, "h", (torch.float32,)), stride_h, objective, lo, hi,
        _dev(center, "center", (torch.uint8,)), _dev(incoming, "incoming", (torch.uint8,)),
        _dev(S, "S", (torch.float32,)), _dev(scales, "scales", (torch.uint8,)),
        _dev(packed, "packed", (torch.uint8,)), _dev(loss, "loss", (torch.float32,)),
        _dev(offset, "offset", (torch.int8,)), _stream(stream)), prepare)


def nvfp4_pack(W, batch, out, inp, ldw, stride_w, scales, S, packed, stream=None, prepare=False):
    G = batch * out * (inp // 16)
    _need(scales, G, "scales")
    _need(packed, G * 8, "packed")
    return _run("nvfp4_pack", (
        _dev(W, "W", (torch.float32, torch.bfloat16)), _wdtype(W), batch, out, inp, ldw, stride_w,
        _dev(scales, "scales", (torch.uint8,)), _dev(S, "S", (torch.float32,)),
        _dev(packed, "packed", (torch.uint8,)), _stream(stream)), prepare)


def nvfp4_quantize_activations_workspace_size(tokens: int, inp: int) -> int:
    return int(_lib.nvfp4_quantize_activations_workspace_size(tokens, inp))


def nvfp4_quantize_activations(X, tokens, inp, ldx, objective, h, lo, hi, rule, S_out, scales,
                               packed, workspace, stream=None, prepare=False):
    G = tokens * (inp // 16)
    _need(scales, G, "scales")
    _need(packed, G * 8, "packed")
    return _run("nvfp4_quantize_activations", (
        _dev(X, "X", (torch.float32, torch.bfloat16)), _wdtype(X), tokens, inp, ldx, objective,
        _dev(h, "h", (torch.float32,)), lo, hi, rule, _dev(S_out, "S_out", (torch.float32,)),
        _dev(scales, "scales", (torch.uint8,)), _dev(packed, "packed", (torch.uint8,)),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)), prepare)


def nvfp4_quantize_activations_noalloc(X, tokens, inp, ldx, objective, h, lo, hi, rule, S_out,
                                       scales, packed, stream=None, prepare=False):
    """nvfp4_quantize_activations without a workspace: the library's own per-GPU scratch (no
    allocation; calls that overlap on one GPU race)."""
    G = tokens * (inp // 16)
    _need(scales, G, "scales")
    _need(packed, G * 8, "packed")
    return _run("nvfp4_quantize_activations_noalloc", (
        _dev(X, "X", (torch.float32, torch.bfloat16)), _wdtype(X), tokens, inp, ldx, objective,
        _dev(h, "h", (torch.float32,)), lo, hi, rule, _dev(S_out, "S_out", (torch.float32,)),
        _dev(scales, "scales", (torch.uint8,)), _dev(packed, "packed", (torch.uint8,)),
        _stream(stream)), prepare)


def nvfp4_gptq_workspace_size(out: int, inp: int) -> int:
    return int(_lib.nvfp4_gptq_workspace_size(out, inp))


def nvfp4_gptq(W, out, inp, ldw, U, h, objective, lo, hi, S, scales, packed, W_final, workspace,
               stream=None, prepare=False):
    _need(scales, out * (inp // 16), "scales")
    _need(packed, out * (inp // 2), "packed")
    _need(U, inp * inp, "U")
    if h is not None:
        _need(h, inp, "h")
    if W_final is not None:
        _need(W_final, out * inp, "W_final")
    return _run("nvfp4_gptq", (
        _dev(W, "W", (torch.float32, torch.bfloat16)), _wdtype(W), out, inp, ldw,
        _dev(U, "U", (torch.float32,)), _dev(h, "h", (torch.float32,)), objective, lo, hi,
        _dev(S, "S", (torch.float32,)), _dev(scales, "scales", (torch.uint8,)),
        _dev(packed, "packed", (torch.uint8,)), _dev(W_final, "W_final", (torch.float32,)),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)), prepare)


def nvfp4_output_error_workspace_size(tokens: int, out: int, inp: int) -> int:
    return int(_lib.nvfp4_output_error_workspace_size(tokens, out, inp))


def nvfp4_output_error(X, tokens, inp, ldx, W, out, ldw, scales, packed, S, err, accumulate,
                       workspace, stream=None, prepare=False):
    _need(err, out, "err")
    return _run("nvfp4_output_error", (
        _dev(X, "X", (torch.bfloat16,)), DTYPE_BF16, tokens, inp, ldx,
        _dev(W, "W", (torch.float32, torch.bfloat16)), _wdtype(W), out, ldw,
        _dev(scales, "scales", (torch.uint8,)), _dev(packed, "packed", (torch.uint8,)),
        _dev(S, "S", (torch.float32,)), _dev(err, "err", (torch.float64,)), int(accumulate),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream)), prepare)


# --- convenience wrappers (allocate outputs with torch, then call the entry points) ----------

def _bmat(W: torch.Tensor):
    """(batch, out, in, ldw, stride_w) of a [out, in] or [batch, out, in] row-major tensor."""
    if W.dim() == 2:
        if W.stride(1) != 1:
            raise ValueError("W rows must be contiguous")
        return 1, W.shape[0], W.shape[1], W.stride(0), W.shape[0] * W.stride(0)
    if W.dim() == 3:
        if W.stride(2) != 1:
            raise ValueError("W rows must be contiguous")
        return W.shape[0], W.shape[1], W.shape[2], W.stride(1), W.stride(0)
    raise ValueError("W must be 2-D or 3-D")


def diag_hessian(X: torch.Tensor, h_acc: torch.Tensor | None = None, accumulate: bool = False,
                 stream=None):
    """h over X [tokens, in]; returns (h_acc float64 [in], h float32 [in])."""
    T, n = X.shape
    if X.stride(1) != 1:
        raise ValueError("X rows must be contiguous")
    if h_acc is None:
        h_acc = torch.zeros(n, dtype=torch.float64, device=X.device)
    h = torch.empty(n, dtype=torch.float32, device=X.device)
    ws = torch.zeros(max(1, nvfp4_diag_hessian_workspace_size(T, n, 1)), dtype=torch.uint8,
                     device=X.device)
    nvfp4_diag_hessian(X, T, n, X.stride(0), h_acc, h, accumulate, ws, stream)
    return h_acc, h


def diag_hessian_batched(X: torch.Tensor, seg_offsets: torch.Tensor,
                         h_acc: torch.Tensor | None = None, accumulate: bool = False, stream=None):
    """Per-segment h over the routed rows of X; returns (h_acc [E, in] f64, h [E, in] f32)."""
    T, n = X.shape
    E = seg_offsets.numel() - 1
    if h_acc is None:
        h_acc = torch.zeros((E, n), dtype=torch.float64, device=X.device)
    h = torch.empty((E, n), dtype=torch.float32, device=X.device)
    ws = torch.zeros(max(1, nvfp4_diag_hessian_workspace_size(T, n, E)), dtype=torch.uint8,
                     device=X.device)
    nvfp4_diag_hessian_batched(X, seg_offsets, E, T, n, X.stride(0), h_acc, h, accumulate, ws,
                               stream)
    return h_acc, h


def layer_statistics(X: torch.Tensor, W: torch.Tensor, rule: int = GS_AMAX_448,
                     h_acc: torch.Tensor | None = None, accumulate: bool = False, stream=None):
    """h over X [tokens, in] and S of W [out, in]; returns (h_acc f64 [in], h f32 [in], S [1])."""
    T, n = X.shape
    o = W.shape[0]
    if X.stride(1) != 1 or W.stride(1) != 1:
        raise ValueError("X and W rows must be contiguous")
    if h_acc is None:
        h_acc = torch.zeros(n, dtype=torch.float64, device=X.device)
    h = torch.empty(n, dtype=torch.float32, device=X.device)
    S = torch.empty(1, dtype=torch.float32, device=X.device)
    ws = torch.empty(max(16, nvfp4_layer_statistics_workspace_size(T, n, o)), dtype=torch.uint8,
                     device=X.device)
    nvfp4_layer_statistics(X, T, n, X.stride(0), h_acc, h, accumulate, W, o, W.stride(0), rule, S,
                           ws, stream)
    return h_acc, h, S


def global_scale(W: torch.Tensor, rule: int = GS_AMAX_448, stream=None) -> torch.Tensor:
    b, o, n, ldw, sw = _bmat(W)
    S = torch.empty(b, dtype=torch.float32, device=W.device)
    ws = torch.zeros(max(1, nvfp4_global_scale_workspace_size(b, o, n)), dtype=torch.uint8,
                     device=W.device)
    nvfp4_global_scale(W, b, o, n, ldw, sw, rule, S, ws, stream)
    return S


def scale_search(W: torch.Tensor, h: torch.Tensor | None, S: torch.Tensor, objective: int,
                 lo: int = -9, hi: int = 6, exhaustive: bool = False, with_stats: bool = True,
                 stream=None):
    """Scale search + pack over W [out, in] or [batch, out, in]; h [in] or [batch, in]."""
    b, o, n, ldw, sw = _bmat(W)
    shp = (o, n // 16) if W.dim() == 2 else (b, o, n // 16)
    dev = W.device
    scales = torch.empty(shp, dtype=torch.uint8, device=dev)
    packed = torch.empty(shp[:-1] + (n // 2,), dtype=torch.uint8, device=dev)
    loss = torch.empty(shp, dtype=torch.float32, device=dev) if with_stats else None
    offset = torch.empty(shp, dtype=torch.int8, device=dev) if with_stats else None
    stride_h = 0
    if objective == WMSE:
        if h is None:
            raise ValueError("WMSE needs h")
        stride_h = h.stride(0) if h.dim() == 2 else 0
    nvfp4_scale_search(W, b, o, n, ldw, sw, 16, h if objective == WMSE else None, stride_h,
                       objective, lo, hi, exhaustive, S, scales, packed, loss, offset, stream)
    return {"scales": scales, "packed": packed, "loss": loss, "offset": offset}


def scale_search_rules(W: torch.Tensor, h: torch.Tensor | None, S: torch.Tensor, rules,
                       with_stats: bool = True, stream=None) -> list[dict]:
    """Several rules (objective, lo, hi, exhaustive) over W [out, in] or [batch, out, in] in one
    call; returns one output dict per rule, as scale_search would."""
    b, o, n, ldw, sw = _bmat(W)
    shp = (o, n // 16) if W.dim() == 2 else (b, o, n // 16)
    dev = W.device
    outs, specs = [], []
    for objective, lo, hi, exhaustive in rules:
        r = {"scales": torch.empty(shp, dtype=torch.uint8, device=dev),
             "packed": torch.empty(shp[:-1] + (n // 2,), dtype=torch.uint8, device=dev),
             "loss": torch.empty(shp, dtype=torch.float32, device=dev) if with_stats else None,
             "offset": torch.empty(shp, dtype=torch.int8, device=dev) if with_stats else None}
        outs.append(r)
        specs.append(dict(r, objective=objective, lo=lo, hi=hi, exhaustive=exhaustive))
    wmse = any(objective == WMSE for objective, *_ in rules)
    if wmse and h is None:
        raise ValueError("WMSE needs h")
    stride_h = (h.stride(0) if h.dim() == 2 else 0) if wmse else 0
    nvfp4_scale_search_rules(W, b, o, n, ldw, sw, 16, h if wmse else None, stride_h, S, specs,
                             stream)
    return outs


def scale_search_scored(W: torch.Tensor, h: torch.Tensor | None, S: torch.Tensor, objective: int,
                        centre_lo: int = -8, stream=None) -> int:
    """Number of (group, code) candidates the exhaustive search scores on these inputs (centre
    block at base + centre_lo: -8 for scale_search's exhaustive mode, the window's lo when a
    16-code window and the exhaustive rule share one scale_search_rules launch)."""
    b, o, n, ldw, sw = _bmat(W)
    stride_h = 0
    if objective == WMSE:
        if h is None:
            raise ValueError("WMSE needs h")
        stride_h = h.stride(0) if h.dim() == 2 else 0
    count = torch.zeros(1, dtype=torch.int64, device=W.device)
    nvfp4_scale_search_scored(W, b, o, n, ldw, sw, 16, h if objective == WMSE else None, stride_h,
                              objective, centre_lo, S, count, stream)
    return int(count.item())


def scale_search_proposal(W: torch.Tensor, h: torch.Tensor | None, S: torch.Tensor, objective: int,
                          center: torch.Tensor, incoming: torch.Tensor | None = None,
                          lo: int = -4, hi: int = 4, with_stats: bool = True, stream=None):
    """Proposal-centred search + pack: window lo..hi around center[...] (uint8, shaped like the
    scales), the incoming codes (or None) scored first and kept on ties."""
    b, o, n, ldw, sw = _bmat(W)
    shp = (o, n // 16) if W.dim() == 2 else (b, o, n // 16)
    dev = W.device
    scales = torch.empty(shp, dtype=torch.uint8, device=dev)
    packed = torch.empty(shp[:-1] + (n // 2,), dtype=torch.uint8, device=dev)
    loss = torch.empty(shp, dtype=torch.float32, device=dev) if with_stats else None
    offset = torch.empty(shp, dtype=torch.int8, device=dev) if with_stats else None
    stride_h = 0
    if objective == WMSE:
        if h is None:
            raise ValueError("WMSE needs h")
        stride_h = h.stride(0) if h.dim() == 2 else 0
    for name, t in (("center", center), ("incoming", incoming)):
        if t is not None and (tuple(t.shape) != shp or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous uint8 tensor of shape {shp}")
    nvfp4_scale_search_proposal(W, b, o, n, ldw, sw, 16, h if objective == WMSE else None,
                                stride_h, objective, lo, hi, center, incoming, S, scales, packed,
                                loss, offset, stream)
    return {"scales": scales, "packed": packed, "loss": loss, "offset": offset}


def quantize_activations(X: torch.Tensor, objective: int = MSE, lo: int = -3, hi: int = 7,
                         rule: int = GS_AMAX_256, h: torch.Tensor | None = None, stream=None):
    """Dynamic per-tensor S and the scale search + pack of X [tokens, in] in two kernels."""
    T, n = X.shape
    if X.stride(1) != 1:
        raise ValueError("X rows must be contiguous")
    dev = X.device
    S = torch.empty(1, dtype=torch.float32, device=dev)
    scales = torch.empty((T, n // 16), dtype=torch.uint8, device=dev)
    packed = torch.empty((T, n // 2), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(16, nvfp4_quantize_activations_workspace_size(T, n)), dtype=torch.uint8,
                     device=dev)
    nvfp4_quantize_activations(X, T, n, X.stride(0), objective, h if objective == WMSE else None,
                               lo, hi, rule, S, scales, packed, ws, stream)
    return {"S": S, "scales": scales, "packed": packed}


def gptq(W: torch.Tensor, U: torch.Tensor, h: torch.Tensor | None, S: torch.Tensor,
         objective: int = WMSE, lo: int = -9, hi: int = 6, with_final: bool = False, stream=None):
    """GPTQ over W [out, in] with the window search as local quantiser (U: upper factor of the
    damped inverse Hessian, float32 [in, in])."""
    o, n = W.shape
    if W.stride(1) != 1:
        raise ValueError("W rows must be contiguous")
    dev = W.device
    scales = torch.empty((o, n // 16), dtype=torch.uint8, device=dev)
    packed = torch.empty((o, n // 2), dtype=torch.uint8, device=dev)
    W_final = torch.empty((o, n), dtype=torch.float32, device=dev) if with_final else None
    ws = torch.empty(max(16, nvfp4_gptq_workspace_size(o, n)), dtype=torch.uint8, device=dev)
    nvfp4_gptq(W, o, n, W.stride(0), U.contiguous(), h if objective == WMSE else None, objective,
               lo, hi, S, scales, packed, W_final, ws, stream)
    return {"scales": scales, "packed": packed, "W_final": W_final}


def output_error(X: torch.Tensor, W: torch.Tensor, packed: torch.Tensor, scales: torch.Tensor,
                 S: torch.Tensor, err: torch.Tensor | None = None, accumulate: bool = False,
                 stream=None) -> torch.Tensor:
    """Per-row layer-output error err[o] = sum_t (X (W - W_hat)^T)[t, o]^2 (float64 [out])."""
    T, n = X.shape
    o = W.shape[0]
    if X.stride(1) != 1 or W.stride(1) != 1:
        raise ValueError("X and W rows must be contiguous")
    if err is None:
        err = torch.empty(o, dtype=torch.float64, device=X.device)
    ws = torch.empty(max(16, nvfp4_output_error_workspace_size(T, o, n)), dtype=torch.uint8,
                     device=X.device)
    nvfp4_output_error(X, T, n, X.stride(0), W, o, W.stride(0), scales.contiguous(),
                       packed.contiguous(), S, err, accumulate, ws, stream)
    return err


def pack(W: torch.Tensor, scales: torch.Tensor, S: torch.Tensor, stream=None) -> torch.Tensor:
    b, o, n, ldw, sw = _bmat(W)
    packed = torch.empty(scales.shape[:-1] + (n // 2,), dtype=torch.uint8, device=W.device)
    nvfp4_pack(W, b, o, n, ldw, sw, scales, S, packed, stream)
    return packed
