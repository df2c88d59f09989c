"""The C-ABI library loads, exports every entry point its header declares, and rejects bad
arguments on the host before anything is enqueued (CPU only: no call here reaches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "block_scale_search_amd", "libnvfp4.so")
HEADER = os.path.join(ROOT, "include", "nvfp4.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libnvfp4.so not built")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared()
    for want in ("nvfp4_diag_hessian", "nvfp4_diag_hessian_batched", "nvfp4_global_scale",
                 "nvfp4_scale_search", "nvfp4_scale_search_rules", "nvfp4_scale_search_proposal",
                 "nvfp4_pack",
                 "nvfp4_output_error", "nvfp4_output_error_workspace_size",
                 "nvfp4_quantize_activations", "nvfp4_quantize_activations_workspace_size",
                 "nvfp4_diag_hessian_finalize", "nvfp4_gptq", "nvfp4_gptq_workspace_size",
                 "nvfp4_status_string",
                 "nvfp4_diag_hessian_workspace_size", "nvfp4_global_scale_workspace_size"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing


def test_binding_covers_every_symbol():
    from block_scale_search_amd import nvfp4
    assert set(_declared()) <= set(nvfp4.EXPORTS)
    assert nvfp4.nvfp4_version().startswith("nvfp4-gfx950")
    for s in range(9):
        assert nvfp4.nvfp4_status_string(s).startswith("NVFP4_")


@pytest.fixture(scope="module")
def lib():
    from block_scale_search_amd import nvfp4
    return nvfp4._lib


FAKE = ctypes.c_void_p(1 << 20)       # 16-byte aligned, never dereferenced: calls fail first
ODD = ctypes.c_void_p((1 << 20) + 4)


def _search(lib, **kw):
    a = dict(W=FAKE, dt=1, batch=1, out=4, inp=64, ldw=64, sw=256, gs=16, h=FAKE, sh=0, obj=1,
             lo=-9, hi=6, exh=0, S=FAKE, sc=FAKE, pk=FAKE, loss=None, off=None)
    a.update(kw)
    return lib.nvfp4_scale_search(a["W"], a["dt"], a["batch"], a["out"], a["inp"], a["ldw"],
                                  a["sw"], a["gs"], a["h"], a["sh"], a["obj"], a["lo"], a["hi"],
                                  a["exh"], a["S"], a["sc"], a["pk"], a["loss"], a["off"], None)


def test_scale_search_rejects_bad_arguments(lib):
    from block_scale_search_amd import nvfp4 as n
    assert _search(lib, gs=32) == n.ERR_ARG
    assert _search(lib, obj=7) == n.ERR_ARG
    assert _search(lib, dt=5) == n.ERR_DTYPE
    assert _search(lib, inp=40, ldw=40) == n.ERR_SHAPE            # in % 16 != 0
    assert _search(lib, ldw=32) == n.ERR_SHAPE                    # ld < in
    assert _search(lib, out=-1) == n.ERR_SHAPE
    assert _search(lib, lo=1) == n.ERR_WINDOW
    assert _search(lib, hi=-1) == n.ERR_WINDOW
    assert _search(lib, lo=-126) == n.ERR_WINDOW
    assert _search(lib, hi=126) == n.ERR_WINDOW
    assert _search(lib, W=None) == n.ERR_NULL
    assert _search(lib, h=None) == n.ERR_NULL                     # WMSE needs h
    assert _search(lib, S=None) == n.ERR_NULL
    assert _search(lib, W=ODD) == n.ERR_ALIGN
    assert _search(lib, ldw=68) == n.ERR_ALIGN                    # bf16 rows of 136 bytes
    assert _search(lib, batch=2, sw=100) == n.ERR_SHAPE           # matrices overlap
    assert _search(lib, out=1 << 26, inp=1 << 10, ldw=1 << 10) == n.ERR_SHAPE
    assert _search(lib, ldw=1 << 62) == n.ERR_SHAPE               # rows x ldw beyond 2^56
    assert _search(lib, out=1 << 20, ldw=1 << 40) == n.ERR_SHAPE
    assert _search(lib, batch=2, sw=1 << 60) == n.ERR_SHAPE       # matrices x stride beyond 2^56
    # empty problems are valid and enqueue nothing
    assert _search(lib, out=0) == n.OK
    assert _search(lib, batch=0) == n.OK
    assert _search(lib, inp=0, ldw=0) == n.OK
    # an exhaustive search ignores the window
    assert _search(lib, exh=1, lo=5, hi=-5, W=None) == n.ERR_NULL


def _scored(lib, **kw):
    a = dict(W=FAKE, dt=1, batch=1, out=4, inp=64, ldw=64, sw=256, gs=16, h=FAKE, sh=0, obj=1,
             clo=-8, S=FAKE, count=FAKE)
    a.update(kw)
    return lib.nvfp4_scale_search_scored(a["W"], a["dt"], a["batch"], a["out"], a["inp"],
                                         a["ldw"], a["sw"], a["gs"], a["h"], a["sh"], a["obj"],
                                         a["clo"], a["S"], a["count"], None)


def test_scale_search_scored_rejects_bad_arguments(lib):
    from block_scale_search_amd import nvfp4 as n
    assert _scored(lib, gs=32) == n.ERR_ARG
    assert _scored(lib, obj=7) == n.ERR_ARG
    assert _scored(lib, clo=1) == n.ERR_WINDOW
    assert _scored(lib, clo=-16) == n.ERR_WINDOW
    assert _scored(lib, dt=5) == n.ERR_DTYPE
    assert _scored(lib, ldw=32) == n.ERR_SHAPE
    assert _scored(lib, W=None) == n.ERR_NULL
    assert _scored(lib, h=None) == n.ERR_NULL                     # WMSE needs h
    assert _scored(lib, S=None) == n.ERR_NULL
    assert _scored(lib, count=None) == n.ERR_NULL
    assert _scored(lib, count=ODD) == n.ERR_ALIGN                 # not 8-byte aligned
    assert _scored(lib, h=ODD) == n.ERR_ALIGN
    assert _scored(lib, out=0) == n.OK                             # empty: nothing enqueued


def _rules(lib, rules=None, n=None, **kw):
    from block_scale_search_amd import nvfp4 as nv
    a = dict(W=FAKE, dt=1, batch=1, out=4, inp=64, ldw=64, sw=256, gs=16, h=FAKE, sh=0, S=FAKE)
    a.update(kw)
    if rules is None:
        rules = [dict(objective=0, lo=-3, hi=7), dict(objective=1, lo=-8, hi=7)]
    arr = (nv.SearchRule * max(1, len(rules)))()
    for k, r in enumerate(rules):
        arr[k] = nv.SearchRule(r.get("objective", 1), r.get("lo", -9), r.get("hi", 6),
                               r.get("exhaustive", 0), r.get("scales", FAKE.value),
                               r.get("packed", FAKE.value), r.get("loss"), r.get("offset"))
    return lib.nvfp4_scale_search_rules(a["W"], a["dt"], a["batch"], a["out"], a["inp"], a["ldw"],
                                        a["sw"], a["gs"], a["h"], a["sh"], a["S"],
                                        None if n == "null" else arr,
                                        len(rules) if n in (None, "null") else n, None)


def test_scale_search_rules_rejects_bad_arguments(lib):
    from block_scale_search_amd import nvfp4 as n
    from block_scale_search_amd.nvfp4 import SearchRule
    lib.nvfp4_scale_search_rules.argtypes = [ctypes.c_void_p, ctypes.c_int] + [ctypes.c_int64] * 5 + [
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
        ctypes.POINTER(SearchRule), ctypes.c_int32, ctypes.c_void_p]
    assert _rules(lib, gs=8) == n.ERR_ARG
    assert _rules(lib, n=0) == n.ERR_ARG
    assert _rules(lib, n=65) == n.ERR_ARG
    assert _rules(lib, n="null") == n.ERR_NULL
    assert _rules(lib, rules=[dict(objective=2)]) == n.ERR_ARG
    assert _rules(lib, rules=[dict(lo=-3, hi=7), dict(lo=1, hi=7)]) == n.ERR_WINDOW
    assert _rules(lib, rules=[dict(exhaustive=1, lo=5, hi=-5)], W=None) == n.ERR_NULL
    assert _rules(lib, h=None) == n.ERR_NULL                        # a WMSE rule needs h
    assert _rules(lib, h=ODD) == n.ERR_ALIGN
    assert _rules(lib, rules=[dict(objective=1), dict(packed=ODD.value)]) == n.ERR_ALIGN
    assert _rules(lib, rules=[dict(objective=1), dict(scales=None)]) == n.ERR_NULL
    assert _rules(lib, dt=3) == n.ERR_DTYPE
    assert _rules(lib, inp=40, ldw=40) == n.ERR_SHAPE
    assert _rules(lib, batch=2, sh=8) == n.ERR_SHAPE                # h rows overlap
    assert _rules(lib, out=0) == n.OK                               # empty: nothing enqueued


def _proposal(lib, **kw):
    a = dict(W=FAKE, dt=1, batch=1, out=4, inp=64, ldw=64, sw=256, gs=16, h=FAKE, sh=0, obj=1,
             lo=-4, hi=4, cen=FAKE, inc=None, S=FAKE, sc=FAKE, pk=FAKE, loss=None, off=None)
    a.update(kw)
    return lib.nvfp4_scale_search_proposal(a["W"], a["dt"], a["batch"], a["out"], a["inp"],
                                           a["ldw"], a["sw"], a["gs"], a["h"], a["sh"], a["obj"],
                                           a["lo"], a["hi"], a["cen"], a["inc"], a["S"], a["sc"],
                                           a["pk"], a["loss"], a["off"], None)


def test_scale_search_proposal_rejects_bad_arguments(lib):
    from block_scale_search_amd import nvfp4 as n
    assert _proposal(lib, gs=8) == n.ERR_ARG
    assert _proposal(lib, obj=2) == n.ERR_ARG
    assert _proposal(lib, lo=1) == n.ERR_WINDOW
    assert _proposal(lib, hi=-2) == n.ERR_WINDOW
    assert _proposal(lib, lo=-126) == n.ERR_WINDOW
    assert _proposal(lib, cen=None) == n.ERR_NULL                 # the proposal is required
    assert _proposal(lib, h=None) == n.ERR_NULL
    assert _proposal(lib, W=ODD) == n.ERR_ALIGN
    assert _proposal(lib, dt=3) == n.ERR_DTYPE
    assert _proposal(lib, inp=40, ldw=40) == n.ERR_SHAPE
    assert _proposal(lib, out=0, cen=None) == n.OK                # empty: nothing enqueued


def test_output_error_rejects_bad_arguments(lib):
    from block_scale_search_amd import nvfp4 as n
    oe = lib.nvfp4_output_error
    need = lib.nvfp4_output_error_workspace_size(256, 4, 64)
    assert need > 0
    ok = dict(X=FAKE, xd=1, T=256, inp=64, ldx=64, W=FAKE, wd=1, out=4, ldw=64, sc=FAKE, pk=FAKE,
              S=FAKE, err=FAKE, acc=0, ws=FAKE, wsb=need)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return oe(a["X"], a["xd"], a["T"], a["inp"], a["ldx"], a["W"], a["wd"], a["out"], a["ldw"],
                  a["sc"], a["pk"], a["S"], a["err"], a["acc"], a["ws"], a["wsb"], None)
    assert call(xd=0) == n.ERR_DTYPE                              # X must be bf16
    assert call(wd=4) == n.ERR_DTYPE
    assert call(inp=40, ldx=40, ldw=40) == n.ERR_SHAPE
    assert call(ldx=60) == n.ERR_SHAPE                            # ldx < in
    assert call(T=-1) == n.ERR_SHAPE
    assert call(T=1 << 40, out=1 << 20, ldw=64) == n.ERR_SHAPE   # tile count >= 2^31
    assert call(T=1 << 20, ldx=1 << 40) == n.ERR_SHAPE           # tokens x ldx beyond 2^56
    assert call(ldw=1 << 60) == n.ERR_SHAPE
    assert call(err=None) == n.ERR_NULL
    assert call(pk=None) == n.ERR_NULL
    assert call(X=ODD) == n.ERR_ALIGN
    assert call(ws=None) == n.ERR_WORKSPACE
    assert call(wsb=need - 1) == n.ERR_WORKSPACE
    assert call(out=0, err=None) == n.OK


def test_quantize_activations_rejects_bad_arguments(lib):
    from block_scale_search_amd import nvfp4 as n
    need = lib.nvfp4_quantize_activations_workspace_size(32, 64)
    assert need > 0

    def call(**kw):
        a = dict(X=FAKE, xd=1, T=32, inp=64, ldx=64, obj=0, h=None, lo=-3, hi=7, rule=1, S=FAKE,
                 sc=FAKE, pk=FAKE, ws=FAKE, wsb=need)
        a.update(kw)
        return lib.nvfp4_quantize_activations(a["X"], a["xd"], a["T"], a["inp"], a["ldx"],
                                              a["obj"], a["h"], a["lo"], a["hi"], a["rule"],
                                              a["S"], a["sc"], a["pk"], a["ws"], a["wsb"], None)
    assert call(obj=3) == n.ERR_ARG
    assert call(rule=2) == n.ERR_ARG                              # a given S is not on-line
    assert call(lo=1) == n.ERR_WINDOW
    assert call(xd=7) == n.ERR_DTYPE
    assert call(inp=40, ldx=40) == n.ERR_SHAPE
    assert call(obj=1) == n.ERR_NULL                              # WMSE needs h
    assert call(sc=None) == n.ERR_NULL
    assert call(X=ODD) == n.ERR_ALIGN
    assert call(wsb=need - 1) == n.ERR_WORKSPACE
    assert call(T=0, X=None) == n.OK


def test_quantize_activations_noalloc_rejects_bad_arguments(lib):
    """The allocation-free variant validates exactly as the workspace call does, before it
    touches the device; its scratch (S slot and at most 512 amax partials) fits the library's
    4096-byte array at every size, the largest included."""
    from block_scale_search_amd import nvfp4 as n

    def call(**kw):
        a = dict(X=FAKE, xd=1, T=32, inp=64, ldx=64, obj=0, h=None, lo=-3, hi=7, rule=1, S=FAKE,
                 sc=FAKE, pk=FAKE)
        a.update(kw)
        return lib.nvfp4_quantize_activations_noalloc(a["X"], a["xd"], a["T"], a["inp"],
                                                      a["ldx"], a["obj"], a["h"], a["lo"],
                                                      a["hi"], a["rule"], a["S"], a["sc"],
                                                      a["pk"], None)
    assert call(obj=3) == n.ERR_ARG
    assert call(rule=2) == n.ERR_ARG
    assert call(lo=1) == n.ERR_WINDOW
    assert call(hi=126) == n.ERR_WINDOW
    assert call(xd=7) == n.ERR_DTYPE
    assert call(inp=40, ldx=40) == n.ERR_SHAPE
    assert call(T=1 << 28, inp=1 << 12, ldx=1 << 12) == n.ERR_SHAPE   # groups >= 2^31
    assert call(obj=1) == n.ERR_NULL
    assert call(pk=None) == n.ERR_NULL
    assert call(X=ODD) == n.ERR_ALIGN
    assert call(T=0, X=None) == n.OK
    for T, inp in ((1, 16), (16, 2048), (8192, 8192), ((1 << 27) - 1, 256)):
        assert lib.nvfp4_quantize_activations_workspace_size(T, inp) <= 4096


def test_hessian_finalize_rejects_bad_arguments(lib):
    from block_scale_search_amd import nvfp4 as n
    f = lib.nvfp4_diag_hessian_finalize
    need = lib.nvfp4_diag_hessian_workspace_size(1000, 64, 1)
    assert f(5, 1000, 64, FAKE, None, 0, FAKE, need, None) == n.ERR_DTYPE
    assert f(1, 1000, 60, FAKE, None, 0, FAKE, need, None) == n.ERR_SHAPE
    assert f(1, 1000, 64, None, None, 0, FAKE, need, None) == n.ERR_NULL
    assert f(1, 1000, 64, ODD, None, 0, FAKE, need, None) == n.ERR_ALIGN
    assert f(1, 1000, 64, FAKE, None, 0, FAKE, need - 8, None) == n.ERR_WORKSPACE
    # deferred partial pass: no outputs, but a workspace is needed
    H = lib.nvfp4_diag_hessian
    assert H(FAKE, 1, 1000, 64, 64, None, None, 0, None, 0, None) == n.ERR_WORKSPACE


def test_gptq_rejects_bad_arguments(lib):
    from block_scale_search_amd import nvfp4 as n
    need = lib.nvfp4_gptq_workspace_size(4, 64)

    def call(**kw):
        a = dict(W=FAKE, wd=1, out=4, inp=64, ldw=64, U=FAKE, h=FAKE, obj=1, lo=-9, hi=6, S=FAKE,
                 sc=FAKE, pk=FAKE, wf=None, ws=FAKE, wsb=need)
        a.update(kw)
        return lib.nvfp4_gptq(a["W"], a["wd"], a["out"], a["inp"], a["ldw"], a["U"], a["h"],
                              a["obj"], a["lo"], a["hi"], a["S"], a["sc"], a["pk"], a["wf"],
                              a["ws"], a["wsb"], None)
    assert call(obj=2) == n.ERR_ARG
    assert call(lo=1) == n.ERR_WINDOW
    assert call(inp=40, ldw=40) == n.ERR_SHAPE
    assert call(U=None) == n.ERR_NULL
    assert call(h=None) == n.ERR_NULL                             # WMSE needs h
    assert call(W=ODD) == n.ERR_ALIGN
    assert call(U=ctypes.c_void_p((1 << 20) + 8)) == n.ERR_ALIGN        # U needs 16 bytes
    assert call(wf=ctypes.c_void_p((1 << 20) + 4)) == n.ERR_ALIGN       # so does W_final
    assert call(wsb=need - 4) == n.ERR_WORKSPACE
    assert call(out=0) == n.OK


def test_pack_and_global_scale_reject_bad_arguments(lib):
    from block_scale_search_amd import nvfp4 as n
    assert lib.nvfp4_pack(FAKE, 1, 1, 4, 40, 40, 160, FAKE, FAKE, FAKE, None) == n.ERR_SHAPE
    assert lib.nvfp4_pack(FAKE, 1, 1, 4, 64, 64, 256, None, FAKE, FAKE, None) == n.ERR_NULL
    assert lib.nvfp4_pack(FAKE, 9, 1, 4, 64, 64, 256, FAKE, FAKE, FAKE, None) == n.ERR_DTYPE
    assert lib.nvfp4_pack(FAKE, 1, 1, 0, 64, 64, 0, None, None, None, None) == n.OK
    assert lib.nvfp4_global_scale(FAKE, 1, 1, 4, 64, 64, 256, 3, FAKE, FAKE, 1 << 20, None) == n.ERR_ARG
    assert lib.nvfp4_global_scale(FAKE, 1, 1, 4, 64, 64, 256, 0, None, FAKE, 1 << 20, None) == n.ERR_NULL
    assert lib.nvfp4_global_scale(FAKE, 1, 1, 4, 64, 64, 256, 0, FAKE, None, 0, None) == n.ERR_WORKSPACE
    assert lib.nvfp4_global_scale(FAKE, 1, 0, 4, 64, 64, 256, 0, None, None, 0, None) == n.OK


def test_diag_hessian_rejects_bad_arguments(lib):
    from block_scale_search_amd import nvfp4 as n
    ws = lib.nvfp4_diag_hessian_workspace_size(1000, 64, 1)
    assert ws >= 2 * 8 * 64                                        # ceil(1000/512) tiles of fp64
    assert lib.nvfp4_diag_hessian_workspace_size(-1, 64, 1) == 0
    assert lib.nvfp4_diag_hessian_workspace_size(1000, 64, 4) > ws  # + per-expert tiles
    H = lib.nvfp4_diag_hessian
    assert H(FAKE, 1, 1000, 60, 64, FAKE, FAKE, 0, FAKE, ws, None) == n.ERR_SHAPE    # in % 8
    assert H(FAKE, 1, 1000, 64, 60, FAKE, FAKE, 0, FAKE, ws, None) == n.ERR_SHAPE    # ldx < in
    assert H(FAKE, 1, 1000, 64, 1 << 50, FAKE, FAKE, 0, FAKE, ws, None) == n.ERR_SHAPE  # span
    assert H(FAKE, 4, 1000, 64, 64, FAKE, FAKE, 0, FAKE, ws, None) == n.ERR_DTYPE
    assert H(None, 1, 1000, 64, 64, FAKE, FAKE, 0, FAKE, ws, None) == n.ERR_NULL
    assert H(FAKE, 1, 1000, 64, 64, None, FAKE, 0, FAKE, ws, None) == n.ERR_NULL
    assert H(FAKE, 1, 1000, 64, 64, FAKE, FAKE, 0, FAKE, ws - 1, None) == n.ERR_WORKSPACE
    assert H(FAKE, 1, 1000, 64, 64, FAKE, FAKE, 0, None, ws, None) == n.ERR_WORKSPACE
    assert H(ODD, 1, 1000, 64, 64, FAKE, FAKE, 0, FAKE, ws, None) == n.ERR_ALIGN
    assert H(FAKE, 1, 1000, 0, 0, None, None, 0, None, 0, None) == n.OK             # in == 0
    B = lib.nvfp4_diag_hessian_batched
    wsb = lib.nvfp4_diag_hessian_workspace_size(1000, 64, 4)
    assert B(FAKE, 1, None, 4, 1000, 64, 64, FAKE, FAKE, 0, FAKE, wsb, None) == n.ERR_NULL
    assert B(FAKE, 1, FAKE, 0, 1000, 64, 64, FAKE, FAKE, 0, FAKE, wsb, None) == n.ERR_SHAPE
    assert B(FAKE, 1, FAKE, 4, 1000, 64, 64, FAKE, FAKE, 0, FAKE, ws, None) == n.ERR_WORKSPACE


def test_layer_statistics_rejects_bad_arguments(lib):
    from block_scale_search_amd import nvfp4 as n
    ws = lib.nvfp4_layer_statistics_workspace_size(1000, 64, 4)
    assert ws >= lib.nvfp4_diag_hessian_workspace_size(1000, 64, 1)   # h partials + amax partials
    assert lib.nvfp4_layer_statistics_workspace_size(-1, 64, 4) == 0

    def call(**kw):
        a = dict(X=FAKE, xd=1, T=1000, inp=64, ldx=64, acc=FAKE, h=FAKE, accum=0, W=FAKE, wd=1,
                 out=4, ldw=64, rule=0, S=FAKE, ws=FAKE, wsb=ws)
        a.update(kw)
        return lib.nvfp4_layer_statistics(a["X"], a["xd"], a["T"], a["inp"], a["ldx"], a["acc"],
                                          a["h"], a["accum"], a["W"], a["wd"], a["out"], a["ldw"],
                                          a["rule"], a["S"], a["ws"], a["wsb"], None)
    assert call(xd=4) == n.ERR_DTYPE
    assert call(wd=4) == n.ERR_DTYPE
    assert call(inp=40, ldx=40, ldw=40) == n.ERR_SHAPE                    # W's in % 16
    assert call(ldx=60) == n.ERR_SHAPE
    assert call(ldx=1 << 50) == n.ERR_SHAPE                               # tokens x ldx span
    assert call(ldw=1 << 60) == n.ERR_SHAPE
    assert call(rule=2) == n.ERR_ARG
    assert call(acc=None) == n.ERR_NULL
    assert call(S=None) == n.ERR_NULL
    assert call(W=None) == n.ERR_NULL
    assert call(X=ODD) == n.ERR_ALIGN
    assert call(W=ODD) == n.ERR_ALIGN
    assert call(wsb=ws - 1) == n.ERR_WORKSPACE
    assert call(ws=None) == n.ERR_WORKSPACE
    assert call(inp=0, ldx=0, ldw=0, X=None, acc=None, W=None, S=None, ws=None, wsb=0) == n.OK


def test_deferred_hessian_slots_never_shrink_with_tokens(lib):
    """A deferred h sequence writes its chunks' row-group sums into workspace slots laid out by
    the first (longest) chunk. A shorter later chunk must use no slot that the first one did not
    initialise, so the slot count of one segment may not decrease as the token count grows.
    The single-segment workspace is slots x in x 8 bytes, so its size shows the count."""
    for inp in (8, 136, 512, 1040, 4096, 8192, 14336, 28672):
        sizes = [lib.nvfp4_diag_hessian_workspace_size(t, inp, 1) for t in range(0, 20001)]
        for t in range(1, len(sizes)):
            assert sizes[t] >= sizes[t - 1], (inp, t)
        # the shapes the advisor found out of order: 1025 vs 1024 and 7936 vs 7680 tokens
        assert sizes[1025] >= sizes[1024] and sizes[7936] >= sizes[7680]


def test_diag_hessian_chunks_rejects_bad_arguments(lib):
    """The one-launch form over token chunks validates every chunk on the host."""
    from block_scale_search_amd import nvfp4 as n
    T = (ctypes.c_int64 * 3)(100, 0, 50)
    need = lib.nvfp4_diag_hessian_chunks_workspace_size(T, 3, 64)
    assert need > 0
    assert lib.nvfp4_diag_hessian_chunks_workspace_size(T, 0, 64) == 0
    assert lib.nvfp4_diag_hessian_chunks_workspace_size(T, 65, 64) == 0

    def call(ptrs=(FAKE, None, FAKE), toks=(100, 0, 50), **kw):
        a = dict(xd=1, inp=64, ldx=64, acc=FAKE, h=FAKE, ws=FAKE, wsb=need)
        a.update(kw)
        P = (ctypes.c_void_p * len(ptrs))(*[None if p is None else p.value for p in ptrs])
        t = (ctypes.c_int64 * len(toks))(*toks)
        return lib.nvfp4_diag_hessian_chunks(P, a["xd"], t, len(toks), a["inp"], a["ldx"],
                                             a["acc"], a["h"], 0, a["ws"], a["wsb"], None)
    assert call(xd=5) == n.ERR_DTYPE
    assert call(ptrs=(), toks=()) == n.ERR_SHAPE
    assert call(inp=60, ldx=64) == n.ERR_SHAPE
    assert call(ldx=32) == n.ERR_SHAPE
    assert call(toks=(100, -1, 50)) == n.ERR_SHAPE
    assert call(ptrs=(FAKE, None, None)) == n.ERR_NULL       # a chunk with tokens needs data
    assert call(ptrs=(FAKE, None, ODD)) == n.ERR_ALIGN
    assert call(acc=None) == n.ERR_NULL
    assert call(wsb=need - 1) == n.ERR_WORKSPACE
    assert call(inp=0) == n.OK
    assert lib.nvfp4_diag_hessian_chunks(None, 1, T, 3, 64, 64, FAKE, FAKE, 0, FAKE, need,
                                         None) == n.ERR_NULL
