"""Benchmark of the NVFP4 block-scale search hot path on one MI355X.

One step = the whole path over one synthetic layer held in HBM:
  diagonal Hessian over X -> global scale of W -> scale search + pack for every mode the
  workload names (attn8b: MSE [-3,7] and WMSE [-8,7]). Two windowed modes of 11 or 16 codes on
  bf16 W run as one nvfp4_scale_search_rules call, whose paired launch reads each group once
  for both (--separate-searches times one nvfp4_scale_search call per mode).
On workloads of one matrix and one token chunk, h and S come from one call
(nvfp4_layer_statistics, two launches; --separate-stats times the two separate calls).
Steps follow one another as the layers of a model would (--schedule pipeline, the default when
two or more input sets rotate): step i + 1's h and S calls (HBM-bound) run on a second stream
while step i's searches (VALU-bound) run on the main stream; every step still does all of its
work, and a set's next h and S wait for the searches that read the set's previous ones. With
--schedule sequential every call of a step runs on one stream, in order, so that every kernel's
time is its own. With --streams 2 (sequential across steps) the h-reduce runs on a second
stream, overlapping the global scale and the searches that do not read h. All streams keep the
default priority.
After the timed steps, the pack-at-given-scales entry point (not part of a step) is timed on
its own over the same layers, with the scale bytes the last search wrote.
Prints one JSON line. `value` is weight-searches per second: every mode run searches each of the
layer's weights once, so a step counts n_weights * n_modes. Several input sets are rotated
(more bytes than the 256 MB MALL) so that every step reads its inputs from HBM.

Per-kernel times come from HIP events recorded on the launch stream around each library call
on every 8th timed step (--events-every; recording them on every step makes the host, not the
GPU, set the step time). The dominant kernel's roofline entry is VALU-bound: algorithmic
lane-operations per launch over the launch time, against the VALU issue peak; `traffic` is read from the committed rocprofv3 counter summary when
its kernel-source hash matches the current sources, else null.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload attn8b] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# VALU issue peak of the build: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.32e12 lane-operations
# per second (a wave64 VALU instruction occupies a 16-lane SIMD for 4 cycles; an fma is one
# operation). The published 157.3 TFLOP/s counts an fma as 2 flops and packed dual-fp32
# instructions, which this build does not emit; 78.6 TFLOP/s is the unpacked fma rate.
VALU_PEAK_TOPS = 39.32
VALU_PEAK_TFLOPS = 78.6
# dense bf16 MFMA peak of MI355X (published, no sparsity)
MFMA_BF16_PEAK_TFLOPS = 2500.0
VALU_PUBLISHED_TFLOPS = 157.3
# algorithmic fp32 operations per element and candidate, one VALU lane-operation each: the
# multiply x = |w| * r, the E2M1 rounding of x, the residual fma, the accumulating fma, and for
# WMSE the weighting multiply h * d
OPS_PER_ELEM_CAND = {"wmse": 5, "mse": 4}
# the same counted as flops (fma = 2)
FLOPS_PER_ELEM_CAND = {"wmse": 7, "mse": 6}

METRIC = "weights/s and HBM GB/s (fraction of peak) for scale search+pack; h-reduce GB/s"
KERNEL_SOURCES = ["block_scale_search_amd/csrc/scale_search.hip",
                  "block_scale_search_amd/csrc/search_device.h",
                  "block_scale_search_amd/csrc/amax_device.h",
                  "block_scale_search_amd/csrc/device_formats.h"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def n_candidates(mode) -> int:
    if mode.exhaustive:
        return 126
    return mode.hi - mode.lo + 1 + (1 if getattr(mode, "proposal", False) else 0)


class Layer:
    """One input set of a workload, resident on the GPU, plus its output buffers."""

    def __init__(self, cfg, k: int, dev):
        import torch

        from block_scale_search_amd import workloads
        cfg_k = type(cfg)(**{**cfg.__dict__, "seed": cfg.seed + 100 * k})
        self.W = workloads.make_weights(cfg_k, dev)
        sigma = workloads.make_sigma(cfg_k, dev)
        self.chunks, self.seg = [], None
        for c in range(workloads.n_chunks(cfg)):
            X, offs = workloads.make_activation_chunk(cfg_k, sigma, c, dev)
            self.chunks.append(X)
            if offs is not None:
                self.seg = torch.from_numpy(offs).to(dev)
        self.batch = cfg.batch
        n = cfg.inp
        E = cfg.batch
        self.h_acc = torch.zeros((E, n) if E > 1 else (n,), dtype=torch.float64, device=dev)
        self.h = torch.empty((E, n) if E > 1 else (n,), dtype=torch.float32, device=dev)
        self.S = torch.empty(E, dtype=torch.float32, device=dev)
        G = cfg.batch * cfg.out * (n // 16)
        self.scales = [torch.empty(G, dtype=torch.uint8, device=dev) for _ in cfg.modes]
        self.packed = [torch.empty(G * 8, dtype=torch.uint8, device=dev) for _ in cfg.modes]


class Runner:
    def __init__(self, cfg, n_sets: int, dev):
        import torch

        from block_scale_search_amd import nvfp4
        self.nv, self.cfg, self.dev = nvfp4, cfg, dev
        self.sets = [Layer(cfg, k, dev) for k in range(n_sets)]
        T = cfg.chunk_tokens or cfg.tokens
        E = cfg.batch
        self.ws_h = torch.zeros(max(1, nvfp4.nvfp4_diag_hessian_workspace_size(T, cfg.inp, E)),
                                dtype=torch.uint8, device=dev)
        self.ws_s = torch.zeros(max(1, nvfp4.nvfp4_global_scale_workspace_size(E, cfg.out, cfg.inp)),
                                dtype=torch.uint8, device=dev)
        self.ws_ls = torch.zeros(max(16, nvfp4.nvfp4_layer_statistics_workspace_size(
            T, cfg.inp, cfg.out)), dtype=torch.uint8, device=dev)
        self.separate_stats = False
        self.separate_searches = False
        self.rule = nvfp4.GS_AMAX_256 if cfg.gs_rule == "amax256" else nvfp4.GS_AMAX_448
        if any(m.proposal for m in cfg.modes):
            # proposal and incoming codes, made once outside the timed steps: the incoming code is
            # the max-abs base code, the proposal is the base code moved by a seeded offset
            from block_scale_search_amd import workloads
            for s in self.sets:
                S = nvfp4.global_scale(s.W, self.rule)
                base = nvfp4.scale_search(s.W, None, S, nvfp4.MSE, 0, 0, with_stats=False)["scales"]
                off = workloads.proposal_offsets(cfg, base.shape, dev)
                s.center = (base.to(torch.int32) + off).clamp(1, 126).to(torch.uint8).contiguous()
                s.incoming = base.contiguous()
            torch.cuda.synchronize()

    def calls(self, s: Layer, aux=None, stage=None):
        """The step as (label, call, stream_role) triples in issue order; each call is a prepared
        C-ABI invocation (arguments marshalled once). With an auxiliary stream, the h-reduce
        runs there ("aux") while the main stream computes the global scale and the searches
        that do not read h; the searches that read h wait for it ("main_after_h"). With a
        stage stream, every call that produces h and S runs there ("stage") and the searches
        run on the main stream."""
        nv, cfg = self.nv, self.cfg
        b, o, n = cfg.batch, cfg.out, cfg.inp
        ldw, sw = n, o * n
        out = []
        import torch
        hs = aux if aux is not None else (stage if stage is not None else
                                          torch.cuda.current_stream())
        h_role = "stage" if stage is not None else "aux"
        deferred = len(s.chunks) > 1 and s.seg is None
        # one matrix, one token chunk, one stream: h and S in one call (two launches)
        fused = aux is None and s.seg is None and len(s.chunks) == 1 and not self.separate_stats
        if fused:
            X = s.chunks[0]
            out.append(("h_reduce+global_scale", nv.nvfp4_layer_statistics(
                X, X.shape[0], n, n, s.h_acc, s.h, False, s.W, o, ldw, self.rule, s.S,
                self.ws_ls, stream=stage, prepare=True), "stage" if stage is not None else "main"))
        for ci, X in enumerate(s.chunks if not fused else []):
            T = X.shape[0]
            if s.seg is not None:
                out.append(("h_reduce", nv.nvfp4_diag_hessian_batched(
                    X, s.seg, b, T, n, n, s.h_acc, s.h, ci > 0, self.ws_h, stream=hs,
                    prepare=True), h_role))
            elif deferred:
                # token chunks of one calibration set: row-group sums accumulate in the
                # workspace, one finalize after the last chunk
                out.append(("h_reduce", nv.nvfp4_diag_hessian(
                    X, T, n, n, None, None, ci > 0, self.ws_h, stream=hs, prepare=True),
                    h_role))
            else:
                out.append(("h_reduce", nv.nvfp4_diag_hessian(
                    X, T, n, n, s.h_acc, s.h, ci > 0, self.ws_h, stream=hs, prepare=True),
                    h_role))
        if deferred:
            out.append(("h_finalize", nv.nvfp4_diag_hessian_finalize(
                s.chunks[0].dtype, s.chunks[0].shape[0], n, s.h_acc, s.h, False, self.ws_h,
                stream=hs, prepare=True), h_role))
        if not fused:
            out.append(("global_scale", nv.nvfp4_global_scale(
                s.W, b, o, n, ldw, sw, self.rule, s.S, self.ws_s, stream=stage, prepare=True),
                "stage" if stage is not None else "main"))
        pair = None if self.separate_searches else paired_modes(cfg)
        if pair is not None:
            # two windowed rules in one call: one launch reads each group once for both
            idx = [cfg.modes.index(m) for m in pair]
            wm_any = any(m.objective == "wmse" for m in pair)
            rules = [dict(objective=nv.WMSE if m.objective == "wmse" else nv.MSE, lo=m.lo,
                          hi=m.hi, exhaustive=False, scales=s.scales[i], packed=s.packed[i])
                     for m, i in zip(pair, idx)]
            out.append((pair_label(pair), nv.nvfp4_scale_search_rules(
                s.W, b, o, n, ldw, sw, 16, s.h if wm_any else None, n if wm_any else 0, s.S,
                rules, prepare=True), "main_after_h" if wm_any else "main"))
        for mi, m in enumerate(cfg.modes):
            wm = m.objective == "wmse"
            if pair is not None and m in pair:
                continue
            if m.proposal:
                out.append((f"search:{m.label}", nv.nvfp4_scale_search_proposal(
                    s.W, b, o, n, ldw, sw, 16, s.h if wm else None, n if wm else 0,
                    nv.WMSE if wm else nv.MSE, m.lo, m.hi, s.center, s.incoming, s.S,
                    s.scales[mi], s.packed[mi], prepare=True),
                    "main_after_h" if wm else "main"))
                continue
            out.append((f"search:{m.label}", nv.nvfp4_scale_search(
                s.W, b, o, n, ldw, sw, 16, s.h if wm else None, n if wm else 0,
                nv.WMSE if wm else nv.MSE, m.lo, m.hi, m.exhaustive, s.S, s.scales[mi],
                s.packed[mi], prepare=True), "main_after_h" if wm else "main"))
        # issue order: aux work first, then main work that does not need h, then the rest
        rank = {"aux": 0, "stage": 0, "main": 1, "main_after_h": 2}
        return sorted(out, key=lambda t: rank[t[2]])


def paired_modes(cfg):
    """The step's two windowed modes when they run as one nvfp4_scale_search_rules call with a
    paired launch (bf16 W, exactly two plain windows of 11 or 16 codes), else None."""
    plain = [m for m in cfg.modes if not m.proposal]
    if len(plain) != 2 or len(plain) != len(cfg.modes):
        return None
    if not str(cfg.w_dtype).endswith("bfloat16"):
        return None
    if any(m.exhaustive or n_candidates(m) not in (11, 16) for m in plain):
        return None
    return plain


def pair_label(modes) -> str:
    return "search:" + "+".join(m.label for m in modes)


def label_modes(cfg, label: str):
    """The modes a search label covers (one mode's "search:A", or the paired call's
    "search:A+B"), else []."""
    one = [m for m in cfg.modes if label == f"search:{m.label}"]
    if one:
        return one
    pair = paired_modes(cfg)
    return pair if pair is not None and label == pair_label(pair) else []


def algorithmic_ops(cfg, label: str) -> int:
    """VALU lane-operations a search call needs by the method's definition (0 for others)."""
    return sum(cfg.n_weights * n_candidates(m) * OPS_PER_ELEM_CAND[m.objective]
               for m in label_modes(cfg, label))


def algorithmic(cfg, label: str):
    """(bytes, flops) one call moves / computes by the method's definition."""
    n_w = cfg.n_weights
    wb = 2 if str(cfg.w_dtype).endswith("bfloat16") else 4
    if label == "h_finalize":
        return cfg.batch * cfg.inp * 12, 0
    if label == "h_reduce":
        T = cfg.chunk_tokens or cfg.tokens
        return T * cfg.inp * 2 + cfg.batch * cfg.inp * 12, 2 * T * cfg.inp
    if label == "global_scale":
        return n_w * wb + 4 * cfg.batch, n_w
    if label == "h_reduce+global_scale":
        T = cfg.chunk_tokens or cfg.tokens
        return T * cfg.inp * 2 + cfg.inp * 12 + n_w * wb + 4, 2 * T * cfg.inp + n_w
    # a search call reads W (and h) once and writes each mode's codes and scale bytes
    modes = label_modes(cfg, label)
    bytes_ = n_w * wb + len(modes) * (n_w // 2 + n_w // 16)
    if any(m.objective == "wmse" for m in modes):
        bytes_ += cfg.batch * cfg.inp * 4
    if any(m.proposal for m in modes):
        bytes_ += 2 * (n_w // 16)      # proposal and incoming code per group
    flops = sum(n_w * n_candidates(m) * FLOPS_PER_ELEM_CAND[m.objective] for m in modes)
    return bytes_, flops


def cpu_time(fn, min_s: float = 2.0):
    """Wall seconds per call of fn (repeated until min_s has passed)."""
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        el = time.perf_counter() - t0
        if el >= min_s:
            return el / n


def host_array(t):
    """A device tensor as the oracle takes it (bf16 as uint16 bit patterns)."""
    import numpy as np
    import torch
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def cpu_baseline(cfg, layer, threads: int):
    """The oracle, as it stands, on a bounded sample of the first input set (the GPU's own
    inputs, copied to the host), projected to the whole step.

    Sample: up to 2^24 weights (whole rows, or whole experts of a batch) and the tokens that feed
    them (the first chunk, or the sampled experts' segments). Passes are repeated until at least
    10 s of wall time. Projection: the h time scales with the step's tokens over the sampled
    tokens, the global-scale and search time with the step's weights over the sampled weights.
    """
    import numpy as np
    import torch

    import oracle

    def host(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    budget = 1 << 24
    S_all = layer.S.cpu().numpy().reshape(-1)
    center = incoming = None
    if cfg.batch == 1:
        R = max(1, min(cfg.out, budget // cfg.inp))
        Ws = [host(layer.W[:R])]
        if hasattr(layer, "center"):
            center, incoming = layer.center[:R].cpu().numpy(), layer.incoming[:R].cpu().numpy()
        Xs = [host(layer.chunks[0])]
        Ss = [float(S_all[0])]
        w_frac = cfg.out / R
        tok_sample = layer.chunks[0].shape[0]
        desc = f"{R} of {cfg.out} rows"
    else:
        E = max(1, min(cfg.batch, budget // (cfg.out * cfg.inp)))
        Ws = [host(layer.W[e]) for e in range(E)]
        seg = layer.seg.cpu().numpy()
        Xs = [host(layer.chunks[0][int(seg[e]):int(seg[e + 1])]) for e in range(E)]
        Ss = [float(S_all[e]) for e in range(E)]
        w_frac = cfg.batch / E
        tok_sample = int(seg[E])
        desc = f"{E} of {cfg.batch} experts"
    tok_frac = cfg.tokens / max(1, tok_sample)
    rule = oracle.GS_AMAX_256 if cfg.gs_rule == "amax256" else oracle.GS_AMAX_448
    mats = list(zip(Ws, Xs, Ss))
    # S is a whole-tensor quantity: with a row sample the searches take the oracle's S of the
    # whole matrix (computed once, untimed); the timed passes still compute S on the sample,
    # whose time is projected like the search's
    S_whole = None
    if cfg.batch == 1 and Ws[0].shape[0] < cfg.out:
        S_whole = oracle.global_scale(host(layer.W), rule)

    t_h = t_s = 0.0
    passes = 0
    first = []            # the first pass's oracle results, for the parity report
    t0 = time.perf_counter()
    while True:
        for W, X, S in mats:
            a = time.perf_counter()
            if cfg.batch == 1:
                acc = None
                acc, h = oracle.diag_hessian(X, acc, threads=threads)
            else:
                acc, h = oracle.diag_hessian(X, None, threads=threads)
            b = time.perf_counter()
            S_o = oracle.global_scale(W, rule)
            if S_whole is not None:
                S_o = S_whole
            res = []
            for m in cfg.modes:
                wm = m.objective == "wmse"
                if m.proposal:
                    res.append(oracle.scale_search_proposal(
                        W, h if wm else None, oracle.WMSE if wm else oracle.MSE, m.lo, m.hi,
                        center, incoming, S_o, threads=threads))
                else:
                    res.append(oracle.scale_search(
                        W, h if wm else None, oracle.WMSE if wm else oracle.MSE, m.lo, m.hi,
                        m.exhaustive, S_o, threads=threads))
            c = time.perf_counter()
            t_h += b - a
            t_s += c - b
            if passes == 0:
                first.append((h, S_o, [r_["scales"] for r_ in res]))
        passes += 1
        if time.perf_counter() - t0 >= 10.0:
            break
    parity = parity_on_sample(cfg, layer, first)
    step_s = (t_h * tok_frac + t_s * w_frac) / passes
    searched = cfg.n_weights * len(cfg.modes)
    return {"value": searched / step_s, "unit": "weights/s", "cores": threads, "kind": "oracle",
            "sample": f"first input set: {desc} and {tok_sample} of {cfg.tokens} tokens, "
                      f"h + global scale + {' + '.join(m.label for m in cfg.modes)}, "
                      f"{passes} passes in {time.perf_counter() - t0:.1f} s on {threads} threads; "
                      f"projected to the whole step (h time x {tok_frac:.3g}, "
                      f"search time x {w_frac:.3g})",
            "parity_on_sample": parity}


def cpu_single_core(cfg, layer):
    """The oracle on one host thread, for the single-matrix workloads up to 2^26 weights: one pass
    over about 2^20 weights (whole rows) and at most 2048 tokens, projected to the whole step by
    the weight and token ratios."""
    import numpy as np

    import oracle

    if cfg.batch != 1 or cfg.n_weights > (1 << 26):
        return None
    R = max(1, min(cfg.out, (1 << 20) // cfg.inp))
    W = host_array(layer.W[:R])
    X = host_array(layer.chunks[0][:2048])
    rule = oracle.GS_AMAX_256 if cfg.gs_rule == "amax256" else oracle.GS_AMAX_448
    S_whole = oracle.global_scale(host_array(layer.W), rule)
    a = time.perf_counter()
    _, h = oracle.diag_hessian(X, None, threads=1)
    b = time.perf_counter()
    oracle.global_scale(W, rule)
    for m in cfg.modes:
        wm = m.objective == "wmse"
        if m.proposal:
            continue
        oracle.scale_search(W, h if wm else None, oracle.WMSE if wm else oracle.MSE, m.lo, m.hi,
                            m.exhaustive, S_whole, threads=1)
    c = time.perf_counter()
    tok_frac = cfg.tokens / X.shape[0]
    w_frac = cfg.out / R
    step_s = (b - a) * tok_frac + (c - b) * w_frac
    return {"value": cfg.n_weights * len(cfg.modes) / step_s, "unit": "weights/s", "cores": 1,
            "sample": f"{R} of {cfg.out} rows and {X.shape[0]} of {cfg.tokens} tokens, one pass, "
                      f"projected (h time x {tok_frac:.3g}, search time x {w_frac:.3g})"}


def parity_on_sample(cfg, layer, first):
    """The GPU's own outputs of the timed steps against the oracle's first pass on the sampled
    rows or experts: h (max relative difference), S (equal or not), and for each mode the
    fraction of groups whose scale byte differs. The GPU searches used the GPU's h, the oracle
    its own, so a WMSE mode's fraction is the flip fraction that h's rounding can cause (0 when
    every h element agrees). Skipped for token-chunked workloads (the oracle sample holds one
    chunk)."""
    import numpy as np
    if len(layer.chunks) != 1:
        return {"note": "not computed: the oracle sample holds one token chunk of several"}
    hg = layer.h.cpu().numpy().reshape(cfg.batch, cfg.inp)
    Sg = layer.S.cpu().numpy().reshape(-1)
    gpr = cfg.inp // 16
    sc = [x.cpu().numpy().reshape(cfg.batch, cfg.out, gpr) for x in layer.scales]
    h_rel, s_eq, mism, groups = 0.0, True, [0] * len(cfg.modes), 0
    for e, (h_o, S_o, scales_o) in enumerate(first):
        ho = np.asarray(h_o, dtype=np.float64).reshape(-1)
        d = np.abs(hg[e].astype(np.float64) - ho) / np.maximum(np.abs(ho), 1e-30)
        h_rel = max(h_rel, float(d.max()))
        s_eq = s_eq and bool(np.float32(S_o) == Sg[e])
        for mi, so in enumerate(scales_o):
            so = np.asarray(so).reshape(-1, gpr)
            mism[mi] += int((sc[mi][e][:so.shape[0]] != so).sum())
        groups += np.asarray(scales_o[0]).size
    return {"groups": groups, "h_max_rel_diff": h_rel, "S_equal": s_eq,
            "scale_mismatch_fraction": {m.label: mism[i] / max(1, groups)
                                        for i, m in enumerate(cfg.modes)}}


def read_traffic(workload: str, kernel_label: str):
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("per_launch_bytes", {}).get(kernel_label)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="attn8b")
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated (0 = enough for >1 GB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--separate-stats", action="store_true",
                    help="h and S as two calls (nvfp4_diag_hessian, nvfp4_global_scale) instead "
                         "of nvfp4_layer_statistics on one-chunk workloads")
    ap.add_argument("--separate-searches", action="store_true",
                    help="one nvfp4_scale_search call per mode instead of one "
                         "nvfp4_scale_search_rules call for a pair of windowed modes")
    ap.add_argument("--streams", type=int, default=1, choices=(1, 2),
                    help="2: h-reduce on a second stream, overlapping the global scale and the "
                         "searches that do not read h")
    ap.add_argument("--schedule", default="pipeline", choices=("pipeline", "sequential"),
                    help="pipeline: the next step's h and S calls run on a second stream while "
                         "this step's searches run (needs two or more input sets and one "
                         "stream); sequential: every call of a step on one stream, in order")
    ap.add_argument("--events-every", type=int, default=8,
                    help="record per-call HIP events on every Nth timed step (1 = all)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--activations", action="store_true",
                    help="also time on-line activation quantisation (dynamic S + MSE [-3,7]) of "
                         "the first token chunk and of a 16-token decode batch, outside the step")
    ap.add_argument("--gptq", action="store_true",
                    help="also time GPTQ with the window search as local quantiser on the first "
                         "layer (U from X^T X of the first token chunk, 1%% damping), outside "
                         "the step")
    ap.add_argument("--output-error", action="store_true",
                    help="also time the layer-output error evaluation (MFMA) of the last mode's "
                         "codes over the first token chunk, outside the step")
    args = ap.parse_args()
    if args.steps < 1 or args.warmup < 0 or args.events_every < 1:
        ap.error("--steps and --events-every must be at least 1, --warmup at least 0")
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); splitting the rows over GPUs "
              "(with one all-reduce of h and of the amax) is a design only and is not launched.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from block_scale_search_amd import workloads
    cfg = workloads.CONFIGS[args.workload]
    dev = torch.device("cuda:0")
    per_set = cfg.n_weights * (2 if str(cfg.w_dtype).endswith("bfloat16") else 4) + \
        cfg.tokens * cfg.inp * 2
    # enough sets for more than 1 GiB of inputs (past the 256 MB MALL), at most 8; the layer
    # pipeline needs at least two
    n_sets = args.sets or max(2 if args.schedule == "pipeline" else 1,
                              min(8, -(-(1 << 30) // per_set)))
    print(f"# workload {cfg.name}: {cfg.description}; {n_sets} input set(s)", file=sys.stderr,
          flush=True)
    runner = Runner(cfg, n_sets, dev)
    runner.separate_stats = args.separate_stats
    runner.separate_searches = args.separate_searches
    torch.cuda.synchronize()

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    main = torch.cuda.current_stream()
    aux = torch.cuda.Stream() if args.streams == 2 else None
    # Layer pipeline: step i + 1's h and S (HBM-bound) run on the stage stream while step i's
    # searches (VALU-bound) run on the main stream. Each input set has its own h, S and outputs;
    # a set's next h and S wait for the searches of its previous use, so two or more sets are
    # needed. Both streams keep the default priority.
    pipelined = args.schedule == "pipeline" and aux is None and n_sets >= 2
    schedule = "pipeline" if pipelined else "sequential"
    stage = torch.cuda.Stream() if pipelined else None
    steps = [runner.calls(s, aux, stage) for s in runner.sets]

    def timed_call(f, st, timed_row):
        if timed_row is None:
            f()
            return
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        f()
        e1.record(st)
        timed_row.append((e0, e1))

    def run_step(calls, timed_row=None):
        """One step. Two streams: the aux stream starts when the step starts (event), the
        main stream waits for the aux work before the searches that read h."""
        if aux is not None:
            aux.wait_stream(main)
        waited = False
        for lab, f, role in calls:
            st = aux if (aux is not None and role == "aux") else main
            if aux is not None and role == "main_after_h" and not waited:
                main.wait_stream(aux)
                waited = True
            timed_call(f, st, timed_row)
        if aux is not None and not waited:
            main.wait_stream(aux)

    ev_stage = [torch.cuda.Event() for _ in range(n_sets)]
    ev_done = [torch.cuda.Event() for _ in range(n_sets)]

    def run_pipelined(first, count, rows=None):
        """Steps first .. first + count - 1 of the set rotation, pipelined. rows (a dict) receives
        each timed step's (start, end) event pairs in call order."""
        def want(i):
            return rows is not None and (i - first) % args.events_every == 0

        def issue_stage(i):
            k = i % n_sets
            if i - first >= n_sets:
                stage.wait_event(ev_done[k])          # the set's previous searches are done
            row = rows.setdefault(i, []) if want(i) else None
            for lab, f, role in steps[k]:
                if role == "stage":
                    timed_call(f, stage, row)
            ev_stage[k].record(stage)

        if count <= 0:
            return
        stage.wait_stream(main)
        issue_stage(first)
        for i in range(first, first + count):
            k = i % n_sets
            if i + 1 < first + count:
                issue_stage(i + 1)
            main.wait_event(ev_stage[k])
            row = rows.setdefault(i, []) if want(i) else None
            for lab, f, role in steps[k]:
                if role != "stage":
                    timed_call(f, main, row)
            ev_done[k].record(main)
        main.wait_stream(stage)

    if pipelined:
        run_pipelined(0, args.warmup)
    else:
        for i in range(args.warmup):
            run_step(steps[i % n_sets])
    torch.cuda.synchronize()

    labels = [lab for lab, _, _ in steps[0]]
    ev = []
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(main)
    if pipelined:
        rows = {}
        run_pipelined(args.warmup, args.steps, rows)
        ev = [rows[i] for i in sorted(rows)]
    else:
        for i in range(args.steps):
            if i % args.events_every:
                run_step(steps[i % n_sets])
                continue
            row = []
            run_step(steps[i % n_sets], row)
            ev.append(row)
    t_end.record(main)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    # pack at given scales: outside the step, timed on its own (events on the main stream)
    nv = runner.nv
    packs = []
    for s_ in runner.sets:
        o_, n_ = cfg.out, cfg.inp
        packs.append(nv.nvfp4_pack(s_.W, cfg.batch, o_, n_, n_, o_ * n_, s_.scales[-1], s_.S,
                                   s_.packed[-1], prepare=True))
    for f in packs:
        f()
    torch.cuda.synchronize()
    p0 = torch.cuda.Event(enable_timing=True)
    p1 = torch.cuda.Event(enable_timing=True)
    reps = 50 * n_sets
    p0.record(main)
    for i in range(reps):
        packs[i % n_sets]()
    p1.record(main)
    torch.cuda.synchronize()
    pack_us = p0.elapsed_time(p1) * 1e3 / reps

    # the h-reduce alone (nvfp4_diag_hessian on each set's X), outside the step, where the step
    # runs it fused with the global scale
    h_alone_us = None
    if any(s_.seg is None and len(s_.chunks) == 1 for s_ in runner.sets[:1]) and \
            not runner.separate_stats:
        hs_ = [nv.nvfp4_diag_hessian(s_.chunks[0], s_.chunks[0].shape[0], cfg.inp, cfg.inp,
                                     s_.h_acc, s_.h, False, runner.ws_h, prepare=True)
               for s_ in runner.sets]
        for f in hs_:
            f()
        torch.cuda.synchronize()
        reps_h = 20 * n_sets
        p0.record(main)
        for i in range(reps_h):
            hs_[i % n_sets]()
        p1.record(main)
        torch.cuda.synchronize()
        h_alone_us = p0.elapsed_time(p1) * 1e3 / reps_h

    # under the layer pipeline the searches share the chip with the next step's h and S; each
    # search call is also timed alone (back to back over the sets, outside the step), which gives
    # the kernel's own rate beside the roofline entry of the timed steps
    search_alone = {}
    if pipelined:
        for lab in dict.fromkeys(l for l in labels if l.startswith("search")):
            fs = [f for st_ in steps for l, f, r in st_ if l == lab]
            reps_s = 10 * len(fs)
            p0.record(main)
            for i in range(reps_s):
                fs[i % len(fs)]()
            p1.record(main)
            torch.cuda.synchronize()
            search_alone[lab] = p0.elapsed_time(p1) * 1e3 / reps_s

    # layer-output error (evaluation, outside the step): X chunk 0 against W and the last
    # mode's codes of each input set
    oe = None
    if args.output_error and cfg.batch == 1:
        T0 = runner.sets[0].chunks[0].shape[0]
        ws_oe = torch.empty(nv.nvfp4_output_error_workspace_size(T0, cfg.out, cfg.inp),
                            dtype=torch.uint8, device=dev)
        errs = [torch.empty(cfg.out, dtype=torch.float64, device=dev) for _ in runner.sets]
        calls_oe = [nv.nvfp4_output_error(s_.chunks[0], T0, cfg.inp, cfg.inp, s_.W, cfg.out,
                                          cfg.inp, s_.scales[-1], s_.packed[-1], s_.S, e_, False,
                                          ws_oe, prepare=True)
                    for s_, e_ in zip(runner.sets, errs)]
        for f in calls_oe:
            f()
        torch.cuda.synchronize()
        reps_oe = max(2 * n_sets, 10)
        p0.record(main)
        for i in range(reps_oe):
            calls_oe[i % n_sets]()
        p1.record(main)
        torch.cuda.synchronize()
        oe_us = p0.elapsed_time(p1) * 1e3 / reps_oe
        flops = 2.0 * T0 * cfg.inp * cfg.out
        oe = {"avg_us": round(oe_us, 2), "tokens": T0, "alg_flops": flops,
              "TFLOP/s": round(flops / oe_us / 1e6, 1),
              "frac_mfma_bf16_2500": round(flops / oe_us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 4),
              "mfma_flops_issued": 2 * flops,
              "note": "E = W - W_hat runs as bf16 E_hi + E_lo, so the MFMAs issue twice the "
                      "algorithmic flops; the time includes the residual split and the "
                      "reduction kernels"}
        if not args.no_cpu:
            import oracle
            Ts = min(T0, 512)
            s_ = runner.sets[0]
            Xh, Wh = host_array(s_.chunks[0][:Ts]), host_array(s_.W)
            ph = host_array(s_.packed[-1]).reshape(cfg.out, cfg.inp // 2)
            sh = host_array(s_.scales[-1]).reshape(cfg.out, cfg.inp // 16)
            Sh = float(s_.S.item())
            t_cpu = cpu_time(lambda: oracle.output_error(Xh, Wh, ph, sh, Sh))
            oe["cpu_oracle"] = {"kind": "oracle", "us_projected": round(t_cpu * 1e6 * T0 / Ts, 1),
                                "sample": f"{Ts} of {T0} tokens, projected by the token ratio",
                                "cores": len(os.sched_getaffinity(0)),
                                "note": "binary64 numpy (its matmul uses the BLAS threads)"}

    # on-line activation quantisation (outside the step): one kernel pair vs global scale +
    # search (three kernels), on a prefill chunk and a decode batch
    acts = None
    if args.activations:
        acts = {}
        X0 = runner.sets[0].chunks[0]
        for name, Xa in (("prefill", X0), ("tokens1024", X0[:1024]), ("tokens256", X0[:256]),
                         ("decode16", X0[:16])):
            Ta, na = Xa.shape
            Sx = torch.empty(1, dtype=torch.float32, device=dev)
            sc = torch.empty(Ta * (na // 16), dtype=torch.uint8, device=dev)
            pk = torch.empty(Ta * (na // 2), dtype=torch.uint8, device=dev)
            wsa = torch.empty(max(16, nv.nvfp4_quantize_activations_workspace_size(Ta, na)),
                              dtype=torch.uint8, device=dev)
            wsg = torch.empty(max(16, nv.nvfp4_global_scale_workspace_size(1, Ta, na)),
                              dtype=torch.uint8, device=dev)
            one = nv.nvfp4_quantize_activations(Xa, Ta, na, na, nv.MSE, None, -3, 7,
                                                nv.GS_AMAX_256, Sx, sc, pk, wsa, prepare=True)
            gs = nv.nvfp4_global_scale(Xa, 1, Ta, na, na, Ta * na, nv.GS_AMAX_256, Sx, wsg,
                                       prepare=True)
            se = nv.nvfp4_scale_search(Xa, 1, Ta, na, na, Ta * na, 16, None, 0, nv.MSE, -3, 7,
                                       False, Sx, sc, pk, prepare=True)

            def timed(fn, reps=200):
                for _ in range(5):
                    fn()
                torch.cuda.synchronize()
                p0.record(main)
                for _ in range(reps):
                    fn()
                p1.record(main)
                torch.cuda.synchronize()
                return p0.elapsed_time(p1) * 1e3 / reps

            us1 = timed(one)
            us2 = timed(lambda: (gs(), se()))
            nbytes = Ta * na * 2 + Ta * na // 2 + Ta * na // 16
            acts[name] = {"tokens": Ta, "in": na, "us": round(us1, 2),
                          "us_global_scale_then_search": round(us2, 2),
                          "GB/s": round(nbytes / us1 / 1e3, 1),
                          "weights/s": Ta * na / (us1 * 1e-6)}
            if not args.no_cpu and Ta <= 1024:
                import oracle
                Xh = host_array(Xa)
                thr = min(16, len(os.sched_getaffinity(0)))

                def cpu_act():
                    So = oracle.global_scale(Xh, oracle.GS_AMAX_256)
                    oracle.scale_search(Xh, None, oracle.MSE, -3, 7, False, So, threads=thr)
                acts[name]["cpu_oracle_us"] = round(cpu_time(cpu_act, 1.0) * 1e6, 1)
                acts[name]["cpu_oracle_threads"] = thr

    # GPTQ (outside the step): the damped inverse-Hessian factor is caller-side preparation
    # (binary64 Gram matrix, inverse and Cholesky), untimed; the library call is timed
    gq = None
    if args.gptq and cfg.batch == 1:
        from block_scale_search_amd import workloads as workloads_mod
        s0 = runner.sets[0]
        Xd = s0.chunks[0].double()
        H = Xd.T @ Xd
        H += 0.01 * torch.diagonal(H).mean() * torch.eye(cfg.inp, dtype=torch.float64, device=dev)
        Ud = torch.linalg.cholesky(torch.cholesky_inverse(torch.linalg.cholesky(H))).T.contiguous()
        U = Ud.float().contiguous()
        hd = torch.diagonal(H).float().contiguous()
        del Xd, H, Ud
        m = next((mm for mm in cfg.modes if mm.objective == "wmse" and not mm.exhaustive
                  and not mm.proposal), None) or workloads_mod.Mode("wmse", -9, 6)
        sc = torch.empty((cfg.out, cfg.inp // 16), dtype=torch.uint8, device=dev)
        pk = torch.empty((cfg.out, cfg.inp // 2), dtype=torch.uint8, device=dev)
        wsq = torch.empty(nv.nvfp4_gptq_workspace_size(cfg.out, cfg.inp), dtype=torch.uint8,
                          device=dev)
        call = nv.nvfp4_gptq(s0.W, cfg.out, cfg.inp, cfg.inp, U, hd, nv.WMSE, m.lo, m.hi, s0.S,
                             sc, pk, None, wsq, prepare=True)
        call()
        torch.cuda.synchronize()
        reps = 3
        p0.record(main)
        for _ in range(reps):
            call()
        p1.record(main)
        torch.cuda.synchronize()
        g_us = p0.elapsed_time(p1) * 1e3 / reps
        n_fma = cfg.out * cfg.inp * (cfg.inp - 1) / 2
        search_ops = cfg.out * cfg.inp * n_candidates(m) * OPS_PER_ELEM_CAND["wmse"]
        gq = {"ms": round(g_us / 1e3, 3), "mode": f"WMSE [{m.lo},{m.hi}]",
              "ordered_fmas": n_fma, "search_lane_ops": search_ops,
              "TOP/s": round((n_fma + search_ops) / g_us / 1e6, 2),
              "frac_valu_issue": round((n_fma + search_ops) / g_us / 1e6 / VALU_PEAK_TOPS, 4),
              "weights/s": cfg.out * cfg.inp / (g_us * 1e-6)}
        if not args.no_cpu:
            import oracle
            rows = min(cfg.out, 128)
            Wh = host_array(s0.W[:rows])
            Uh, hh = U.cpu().numpy(), hd.cpu().numpy()
            Sh = float(s0.S.item())
            thr = min(16, len(os.sched_getaffinity(0)))
            t_cpu = cpu_time(lambda: oracle.gptq(Wh, Uh, hh, oracle.WMSE, m.lo, m.hi, Sh,
                                                 threads=thr))
            gq["cpu_oracle"] = {"kind": "oracle", "ms_projected": round(t_cpu * 1e3 * cfg.out / rows, 1),
                                "sample": f"{rows} of {cfg.out} rows (rows are independent), "
                                          "projected by the row ratio",
                                "cores": thr}

    per_label = {}
    for row in ev:
        for lab, (e0, e1) in zip(labels, row):
            per_label.setdefault(lab, []).append(e0.elapsed_time(e1) * 1e3)  # us
    kernels = {}
    for lab, us in per_label.items():
        us_avg = sum(us) / len(us)
        nb, nf = algorithmic(cfg, lab)
        k = {"avg_us": round(us_avg, 3), "calls_per_step": labels.count(lab),
             "alg_bytes": nb, "GB/s": round(nb / us_avg / 1e3, 1),
             "frac_hbm": round(nb / us_avg / 1e3 / HBM_PEAK_GBS, 4)}
        if lab.startswith("search"):
            k["weights/s"] = cfg.n_weights * len(label_modes(cfg, lab)) / (us_avg * 1e-6)
            if "exhaustive" in lab:
                # exact pruning skips candidates that provably lose, so the 126-candidate flop
                # count over the time is an equivalent rate, not a roofline figure
                k["TFLOP/s_126_equivalent"] = round(nf / us_avg / 1e6, 2)
            else:
                no = algorithmic_ops(cfg, lab)
                k["TOP/s"] = round(no / us_avg / 1e6, 2)
                k["frac_valu_issue"] = round(no / us_avg / 1e6 / VALU_PEAK_TOPS, 4)
                k["TFLOP/s"] = round(nf / us_avg / 1e6, 2)
        kernels[lab] = k
    wb = 2 if str(cfg.w_dtype).endswith("bfloat16") else 4
    pack_bytes = cfg.n_weights * wb + cfg.n_weights // 2 + cfg.n_weights // 16
    if h_alone_us is not None:
        xb = (cfg.chunk_tokens or cfg.tokens) * cfg.inp * 2
        kernels["h_reduce alone (outside the step)"] = {
            "avg_us": round(h_alone_us, 3), "x_bytes": xb,
            "GB/s": round(xb / h_alone_us / 1e3, 1),
            "frac_hbm": round(xb / h_alone_us / 1e3 / HBM_PEAK_GBS, 4)}
    kernels["pack (outside the step)"] = {
        "avg_us": round(pack_us, 3), "calls_per_step": 0, "alg_bytes": pack_bytes,
        "GB/s": round(pack_bytes / pack_us / 1e3, 1),
        "frac_hbm": round(pack_bytes / pack_us / 1e3 / HBM_PEAK_GBS, 4)}
    # the roofline entry is the windowed search with the largest share of the step (the
    # exhaustive mode's pruned work has no fixed flop count)
    dom = max((l for l in kernels if l.startswith("search") and "exhaustive" not in l),
              key=lambda l: kernels[l]["avg_us"] * kernels[l]["calls_per_step"])
    nb, nf = algorithmic(cfg, dom)
    no = algorithmic_ops(cfg, dom)
    us_dom = kernels[dom]["avg_us"]
    achieved = no / us_dom / 1e6
    roofline = {"bound": "alu", "kernel": dom, "achieved": round(achieved, 2),
                "peak": VALU_PEAK_TOPS, "unit": "TOP/s (VALU lane-operations)",
                "frac": round(achieved / VALU_PEAK_TOPS, 4),
                "traffic": read_traffic(cfg.name, dom),
                "alg_ops_per_launch": no,
                "achieved_TFLOP/s": round(nf / us_dom / 1e6, 2),
                "frac_of_unpacked_78.6_TFLOP/s": round(nf / us_dom / 1e6 / VALU_PEAK_TFLOPS, 4),
                "frac_of_published_157.3_TFLOP/s": round(nf / us_dom / 1e6 / VALU_PUBLISHED_TFLOPS, 4),
                "alg_bytes_per_launch": nb, "alg_flops_per_launch": nf,
                "hbm_GB/s_algorithmic": kernels[dom]["GB/s"],
                "hbm_frac_algorithmic": kernels[dom]["frac_hbm"]}
    if dom in search_alone:
        ua = search_alone[dom]
        roofline["alone"] = {
            "avg_us": round(ua, 3), "achieved": round(no / ua / 1e6, 2),
            "frac": round(no / ua / 1e6 / VALU_PEAK_TOPS, 4),
            "note": "the same call back to back outside the timed steps; in the steps it shares "
                    "the compute units with the next step's h and S"}

    cpu = None
    if not args.no_cpu:
        threads = min(16, len(os.sched_getaffinity(0)))
        cpu = cpu_baseline(cfg, runner.sets[0], threads)
        one = cpu_single_core(cfg, runner.sets[0])
        if one is not None:
            cpu["single_core"] = one

    # the h stage of a step: every chunk's call plus the deferred finalize, over X's bytes; with
    # the fused call, h and S together over the bytes of X and W
    x_bytes = cfg.tokens * cfg.inp * 2
    if "h_reduce+global_scale" in kernels:
        h_us = kernels["h_reduce+global_scale"]["avg_us"]
        st_bytes = algorithmic(cfg, "h_reduce+global_scale")[0]
        h_stage_gbs = round(st_bytes / h_us / 1e3, 1)
        kernels["h+S stage (one call, X and W bytes)"] = {
            "us_per_step": round(h_us, 2), "bytes": st_bytes, "GB/s": h_stage_gbs,
            "frac_hbm": round(h_stage_gbs / HBM_PEAK_GBS, 4)}
    else:
        h_us = kernels["h_reduce"]["avg_us"] * kernels["h_reduce"]["calls_per_step"]
        if "h_finalize" in kernels:
            h_us += kernels["h_finalize"]["avg_us"]
        h_stage_gbs = round(x_bytes / h_us / 1e3, 1)
        kernels["h_stage (all chunks + finalize)"] = {
            "us_per_step": round(h_us, 2), "x_bytes": x_bytes, "GB/s": h_stage_gbs,
            "frac_hbm": round(h_stage_gbs / HBM_PEAK_GBS, 4)}

    searched = cfg.n_weights * len(cfg.modes)
    line = {
        "metric": METRIC,
        "value": searched / (ms_per_step * 1e-3),
        "unit": "weights/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; stands in for the pages' calibration sets and checkpoints)",
        "config": {"workload": cfg.description, "name": cfg.name,
                   "modes": [m.label for m in cfg.modes], "global_scale": cfg.gs_rule,
                   "weights_per_step": searched, "input_sets_rotated": n_sets,
                   "streams": args.streams, "schedule": schedule},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "h_reduce_GB/s" if "h_reduce" in kernels else "h_and_global_scale_GB/s": h_stage_gbs,
        **({"h_reduce_alone_GB/s": kernels["h_reduce alone (outside the step)"]["GB/s"]}
           if "h_reduce alone (outside the step)" in kernels else {}),
    }
    if oe is not None:
        line["output_error"] = oe
    if acts is not None:
        line["activations"] = acts
    if gq is not None:
        line["gptq"] = gq
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
