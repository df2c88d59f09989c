"""CPU oracle for NVFP4 per-group E4M3 block-scale search.

TEST INFRASTRUCTURE ONLY. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU library
(``block_scale_search_amd``) never imports it, shares no code with it, and fails loudly
if its own HIP extension is missing.

The arithmetic lives in ``nvfp4_ref.c`` (plain C, built with ``gcc -O2
-ffp-contract=off -fopenmp``); this module only marshals numpy arrays. bf16 data is passed
as raw ``uint16`` bit patterns. Every function states the passage it follows in the C
source. Parity status of each part:

* E2M1 rounding, E4M3 encode/decode, h, global scale, base code, candidate loss and argmin:
  pinned by the checks in ``tests/test_oracle_*.py`` (closed forms, a library routine,
  exact-rational recomputation, brute force, and the bounds the ScaleSweep page states).
* Dequantisation and the layer-output error: pinned by the closed forms in
  ``tests/test_oracle_output_error.py`` (quantised weights give zero error, identity
  activations give the squared residual norm, scaling X by 2 multiplies by 4) and brute force
  in exact rationals on a tiny layer.
* Proposal-centred search: pinned by exact-rational recomputation of its candidate list, the
  reduction to the plain window search (centre = base, no incoming code), the retain-on-tie
  rule (h = 0) and the no-increase guarantee against the incoming scale.
* Nibble order inside a byte (low nibble = even element) and the binary32 operation order:
  conventions the pages do not fix. The nibble contents are pinned by a dequantisation round
  trip; the byte order itself is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_ref.c")
_LIB_PATH = os.path.join(_HERE, "libnvfp4_ref.so")

F32, BF16 = 0, 1
MSE, WMSE = 0, 1
GS_AMAX_448, GS_AMAX_256, GS_GIVEN = 0, 1, 2

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (host only)."""
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-o", _LIB_PATH + ".tmp", _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build(force=True)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.ref_e2m1_index.argtypes = [ctypes.c_float]
    lib.ref_e2m1_index.restype = I
    lib.ref_e2m1_level.argtypes = [I]
    lib.ref_e2m1_level.restype = ctypes.c_float
    lib.ref_e4m3_value.argtypes = [I]
    lib.ref_e4m3_value.restype = ctypes.c_double
    lib.ref_e4m3_encode.argtypes = [ctypes.c_float]
    lib.ref_e4m3_encode.restype = I
    lib.ref_e2m1_index_many.argtypes = [P, I64, P]
    lib.ref_e4m3_encode_many.argtypes = [P, I64, P]
    lib.ref_diag_hessian.argtypes = [P, I, I64, I64, I64, P, I, P, I]
    lib.ref_diag_hessian.restype = I
    lib.ref_global_scale.argtypes = [P, I, I64, I64, I64, I, ctypes.c_float, P]
    lib.ref_global_scale.restype = I
    lib.ref_scale_tables.argtypes = [ctypes.c_float, P, P]
    lib.ref_scale_tables.restype = I
    lib.ref_scale_search.argtypes = [P, I, I64, I64, I64, P, I, I, I, I, ctypes.c_float,
                                     P, P, P, P, I]
    lib.ref_scale_search.restype = I
    lib.ref_scale_search_proposal.argtypes = [P, I, I64, I64, I64, P, I, I, I, P, P,
                                              ctypes.c_float, P, P, P, P, I]
    lib.ref_scale_search_proposal.restype = I
    lib.ref_gptq.argtypes = [P, I, I64, I64, I64, P, P, I, I, I, ctypes.c_float, P, P, P, I]
    lib.ref_gptq.restype = I
    lib.ref_dequant.argtypes = [P, P, I64, I64, ctypes.c_float, P]
    lib.ref_dequant.restype = I
    lib.ref_group_candidates.argtypes = [P, P, ctypes.c_float, I, I, I, P, P]
    lib.ref_group_candidates.restype = I
    lib.ref_pack.argtypes = [P, I, I64, I64, I64, P, ctypes.c_float, P, I]
    lib.ref_pack.restype = I
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError("oracle inputs are float32 or bf16 bit patterns (uint16)")


def default_threads() -> int:
    return max(1, min(16, len(os.sched_getaffinity(0))))


# --- element formats -------------------------------------------------------------------------

def e2m1_index(x) -> np.ndarray:
    """E2M1 round-to-nearest-even index of non-negative float32 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    _load().ref_e2m1_index_many(_ptr(x), x.size, _ptr(out))
    return out


def e2m1_level(index: int) -> float:
    return float(_load().ref_e2m1_level(int(index)))


def e4m3_value(code: int) -> float:
    return float(_load().ref_e4m3_value(int(code)))


def e4m3_encode(s) -> np.ndarray:
    """E4M3 round-to-nearest-even code (saturating at 448) of non-negative float32 values."""
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.empty(s.shape, dtype=np.uint8)
    _load().ref_e4m3_encode_many(_ptr(s), s.size, _ptr(out))
    return out


def scale_tables(S: float):
    eff = np.zeros(127, dtype=np.float32)
    rcp = np.zeros(127, dtype=np.float32)
    rc = _load().ref_scale_tables(ctypes.c_float(S), _ptr(eff), _ptr(rcp))
    if rc != 0:
        raise ValueError("global scale gives non-finite effective scales")
    return eff, rcp


# --- the hot path ----------------------------------------------------------------------------

def diag_hessian(X: np.ndarray, acc: np.ndarray | None = None, threads: int | None = None):
    """h = sum_t x_t^2 per column, fp64 sum in token order; returns (acc fp64, h fp32).

    ``X`` is [tokens, in] float32 or bf16 bits; if ``acc`` is given the sum continues from it.
    """
    X = np.ascontiguousarray(X)
    T, n = X.shape
    accumulate = acc is not None
    acc = np.zeros(n, dtype=np.float64) if acc is None else np.ascontiguousarray(acc, np.float64).copy()
    h = np.empty(n, dtype=np.float32)
    rc = _load().ref_diag_hessian(_ptr(X), _dtype_code(X), T, n, n, _ptr(acc), int(accumulate),
                                  _ptr(h), threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle diag_hessian failed ({rc})")
    return acc, h


def global_scale(W: np.ndarray, rule: int, given: float = 1.0) -> float:
    W = np.ascontiguousarray(W)
    out, n = W.shape
    S = np.zeros(1, dtype=np.float32)
    rc = _load().ref_global_scale(_ptr(W), _dtype_code(W), out, n, n, rule, ctypes.c_float(given),
                                  _ptr(S))
    if rc != 0:
        raise ValueError(f"oracle global_scale failed ({rc})")
    return float(S[0])


def scale_search(W: np.ndarray, h: np.ndarray | None, objective: int, lo: int = -9, hi: int = 6,
                 exhaustive: bool = False, S: float = 1.0, threads: int | None = None):
    """Per-group scale search + pack over W[out, in]; returns dict of numpy outputs."""
    W = np.ascontiguousarray(W)
    out, n = W.shape
    hh = None if h is None else np.ascontiguousarray(h, dtype=np.float32)
    scales = np.empty((out, n // 16), dtype=np.uint8)
    packed = np.empty((out, n // 2), dtype=np.uint8)
    loss = np.empty((out, n // 16), dtype=np.float32)
    offset = np.empty((out, n // 16), dtype=np.int8)
    rc = _load().ref_scale_search(_ptr(W), _dtype_code(W), out, n, n, _ptr(hh), objective, lo, hi,
                                  int(exhaustive), ctypes.c_float(S), _ptr(scales), _ptr(packed),
                                  _ptr(loss), _ptr(offset), threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle scale_search failed ({rc})")
    return {"scales": scales, "packed": packed, "loss": loss, "offset": offset}


def scale_search_proposal(W: np.ndarray, h: np.ndarray | None, objective: int, lo: int, hi: int,
                          center: np.ndarray, incoming: np.ndarray | None, S: float,
                          threads: int | None = None):
    """Proposal-centred search (Replay the Curvature App. D.2): the incoming code (if valid),
    then clamp(center + o) for o = lo..hi; strict improvement only, so ties keep the incoming
    code. ``center`` / ``incoming`` are uint8 [out, in/16]. Returns the same dict as
    ``scale_search`` with offset = c* - clamp(center)."""
    W = np.ascontiguousarray(W)
    out, n = W.shape
    hh = None if h is None else np.ascontiguousarray(h, dtype=np.float32)
    cen = np.ascontiguousarray(center, dtype=np.uint8).reshape(out, n // 16)
    inc = None if incoming is None else np.ascontiguousarray(incoming, dtype=np.uint8).reshape(out, n // 16)
    scales = np.empty((out, n // 16), dtype=np.uint8)
    packed = np.empty((out, n // 2), dtype=np.uint8)
    loss = np.empty((out, n // 16), dtype=np.float32)
    offset = np.empty((out, n // 16), dtype=np.int8)
    rc = _load().ref_scale_search_proposal(_ptr(W), _dtype_code(W), out, n, n, _ptr(hh), objective,
                                           lo, hi, _ptr(cen), _ptr(inc), ctypes.c_float(S),
                                           _ptr(scales), _ptr(packed), _ptr(loss), _ptr(offset),
                                           threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle scale_search_proposal failed ({rc})")
    return {"scales": scales, "packed": packed, "loss": loss, "offset": offset}


def group_candidates(w16, h16, S: float, lo: int = -9, hi: int = 6, exhaustive: bool = False):
    """(base code, candidate codes, candidate losses) of one group, in loop order."""
    w16 = np.ascontiguousarray(w16, dtype=np.float32)
    hh = None if h16 is None else np.ascontiguousarray(h16, dtype=np.float32)
    count = 126 if exhaustive else hi - lo + 1
    codes = np.zeros(count, dtype=np.int32)
    losses = np.zeros(count, dtype=np.float32)
    b = _load().ref_group_candidates(_ptr(w16), _ptr(hh), ctypes.c_float(S), lo, hi,
                                     int(exhaustive), _ptr(codes), _ptr(losses))
    if b < 0:
        raise ValueError("bad global scale")
    return b, codes, losses


def pack(W: np.ndarray, scales: np.ndarray, S: float, threads: int | None = None) -> np.ndarray:
    W = np.ascontiguousarray(W)
    out, n = W.shape
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    packed = np.empty((out, n // 2), dtype=np.uint8)
    rc = _load().ref_pack(_ptr(W), _dtype_code(W), out, n, n, _ptr(scales), ctypes.c_float(S),
                          _ptr(packed), threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle pack failed ({rc})")
    return packed


def gptq(W: np.ndarray, U: np.ndarray, h: np.ndarray | None, objective: int, lo: int, hi: int,
         S: float, threads: int | None = None):
    """GPTQ with the window search as local quantiser (H-Scale App. B). U: the upper factor of
    the damped inverse Hessian, float32 [in, in]. Returns scales, packed and the updated
    binary32 weights W_final."""
    W = np.ascontiguousarray(W)
    out, n = W.shape
    U = np.ascontiguousarray(U, dtype=np.float32)
    hh = None if h is None else np.ascontiguousarray(h, dtype=np.float32)
    scales = np.empty((out, n // 16), dtype=np.uint8)
    packed = np.empty((out, n // 2), dtype=np.uint8)
    W_final = np.empty((out, n), dtype=np.float32)
    rc = _load().ref_gptq(_ptr(W), _dtype_code(W), out, n, n, _ptr(U), _ptr(hh), objective, lo,
                          hi, ctypes.c_float(S), _ptr(scales), _ptr(packed), _ptr(W_final),
                          threads or default_threads())
    if rc != 0:
        raise ValueError(f"oracle gptq failed ({rc})")
    return {"scales": scales, "packed": packed, "W_final": W_final}


def dequant(packed: np.ndarray, scales: np.ndarray, S: float) -> np.ndarray:
    """Binary32 dequantised weights [out, in] from packed codes [out, in/2] and scales."""
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    out, half = packed.shape
    w_hat = np.empty((out, 2 * half), dtype=np.float32)
    rc = _load().ref_dequant(_ptr(packed), _ptr(scales), out, 2 * half, ctypes.c_float(S),
                             _ptr(w_hat))
    if rc != 0:
        raise ValueError(f"oracle dequant failed ({rc})")
    return w_hat


def output_error(X: np.ndarray, W: np.ndarray, packed: np.ndarray, scales: np.ndarray,
                 S: float) -> np.ndarray:
    """Per-output-row layer-output error err[o] = sum_t (sum_i x_ti (w_oi - w_hat_oi))^2
    (H-Scale §3: the quantised layer's output against the original's on calibration inputs).

    Everything in binary64: x and w are exact in binary64, w_hat is the binary32 dequantised
    weight, the residual w - w_hat is exact in binary64, and the product is a binary64 matmul
    (a library primitive as one step), then the squares are summed over tokens."""
    def f64(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:            # bf16 bit patterns
            return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        return a.astype(np.float64)
    E = f64(W) - dequant(packed, scales, S).astype(np.float64)
    Y = f64(X) @ E.T
    return (Y * Y).sum(axis=0)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """[.., in/2] bytes -> [.., in] nibbles (low nibble = even element)."""
    lo = packed & 0x0F
    hi = packed >> 4
    return np.stack([lo, hi], axis=-1).reshape(*packed.shape[:-1], packed.shape[-1] * 2)
