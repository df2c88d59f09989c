"""Benchmark of the NVFP4 block-scale search hot path on one MI355X.

One step = the whole path over one synthetic layer held in HBM, or over both matrices of the
70B-shaped MLP pair (the default workload, `mlp70b`): for each matrix,
  diagonal Hessian over its X (8192-token chunks: deferred partial sums plus one finalize; one
  chunk: one call that also computes the global scale) -> global scale of W -> scale search +
  pack for every mode of the workload (mlp70b: WMSE [-9,6] and the exhaustive 126-code mode).
Two modes run as one nvfp4_scale_search_rules call and one launch where the library fuses them:
a 16-code window with the exhaustive mode of its objective (the window is the exhaustive
search's first block of codes), or two windows of 11 or 16 codes on bf16 W (one read of each
group for both); --separate-searches times one call per mode.
Consecutive layers follow one another as in a model (--schedule pipeline, the default): layer
j + 1's h and S calls (HBM-bound) run on a second stream while layer j's searches (VALU-bound)
run on the main stream; every layer still does all of its work, and an input set's next h and
S wait for the searches that read its previous ones. --schedule sequential runs every call on
one stream, in order, so that every kernel's time is its own. Both streams keep the default
priority. Several input sets rotate, so that every step reads its inputs from HBM.

Prints one JSON line. `value` is layer weights per second: the weights of the step's matrices
over the step time (each weight is searched once per mode; `weight_searches_per_s` counts those).
Per-call times come from HIP events recorded on the launch stream around each library call on
every 8th timed step (--events-every). The roofline entry is the search call with the largest
share of the step: its flops per launch (multiply, residual fma, weighting multiply and
accumulating fma per element and candidate scored) over its average launch time, against the
published 157.3 TFLOP/s fp32 vector peak; the lane-issue fraction and the HBM fraction sit
beside it. A window scores every candidate; the exhaustive mode skips the codes its lower
bounds prove to lose, so its candidates are counted on the same inputs with
nvfp4_scale_search_scored (outside the timing), and its 126-code-equivalent rate is given too.
`traffic` is read from the committed rocprofv3 counter summary while its kernel-source hash
matches the current sources, else null.
After the timed steps, the pack-at-given-scales entry point, each layer's h stage and each
search call are timed again on their own, back to back over the input sets.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mlp70b] [--no-cpu]
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
# fp32 vector peak of MI355X: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz = 39.32e12 lane-operations/s;
# an fma counts 2 flops (78.6 TFLOP/s) and packed dual-fp32 instructions double it again to the
# published 157.3 TFLOP/s. The build emits no packed fp32, so 78.6 TFLOP/s is its own ceiling.
VALU_PUBLISHED_TFLOPS = 157.3
VALU_ISSUE_TOPS = 39.32
VALU_UNPACKED_TFLOPS = 78.6
# dense bf16 MFMA peak of MI355X (published, no sparsity)
MFMA_BF16_PEAK_TFLOPS = 2500.0
# the method's flops per element and candidate: x = |w| r (1), the residual fma (2), for WMSE
# the weighting multiply h d (1), the accumulating fma (2). The E2M1 rounding is a conversion,
# not a flop.
FLOPS_PER_ELEM_CAND = {"wmse": 6, "mse": 5}
# VALU lane-operations per element and candidate: the same with the rounding as one operation
# and an fma as one operation
OPS_PER_ELEM_CAND = {"wmse": 5, "mse": 4}

METRIC = "weights/s and HBM GB/s (fraction of peak) for scale search+pack; h-reduce GB/s"
KERNEL_SOURCES = ["block_scale_search_amd/csrc/scale_search.hip",
                  "block_scale_search_amd/csrc/search_device.h",
                  "block_scale_search_amd/csrc/amax_device.h",
                  "block_scale_search_amd/csrc/device_formats.h"]
DEFAULT_WORKLOAD = "mlp70b"


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


def is_bf16(cfg) -> bool:
    return str(cfg.w_dtype).endswith("bfloat16")


def fused_modes(cfg):
    """A 16-code window and the exhaustive mode of the same objective, which one
    nvfp4_scale_search_rules call runs as one launch (the exhaustive search's first block is the
    window), else None."""
    for w in cfg.modes:
        if w.proposal or w.exhaustive or n_candidates(w) != 16:
            continue
        for e in cfg.modes:
            if e.exhaustive and e.objective == w.objective:
                return [w, e]
    return None


def paired_modes(cfg):
    """The two modes that run as one nvfp4_scale_search_rules call and one launch: a 16-code
    window with the exhaustive mode of its objective (fused launch), or exactly two plain
    windows of 11 or 16 codes on bf16 W (paired launch); else None."""
    fused = fused_modes(cfg)
    if fused is not None:
        return fused
    plain = [m for m in cfg.modes if not m.proposal]
    if len(plain) != 2 or len(plain) != len(cfg.modes) or not is_bf16(cfg):
        return None
    if any(m.exhaustive or n_candidates(m) not in (11, 16) for m in plain):
        return None
    return plain


def nested_windows(modes) -> bool:
    """Two windows the library scans as one (k_scale_search_nested): one of 16 codes holding the
    other, which has 11 codes ending where the outer ends, or the same 16 codes."""
    if len(modes) != 2 or any(m.exhaustive or m.proposal for m in modes):
        return False
    for o, i in (modes, modes[::-1]):
        if n_candidates(o) == 16 and (i.lo - o.lo, n_candidates(i)) in ((5, 11), (0, 16)):
            return True
    return False


def kernel_name(cfg, label: str) -> str:
    modes = label_modes(cfg, label)
    what = base_label(label)[len("search:"):]
    if any(m.exhaustive for m in modes):
        return f"k_scale_search_exhaustive {what}" + (" (one fused launch)" if len(modes) > 1
                                                      else "")
    if nested_windows(modes):
        return f"k_scale_search_nested {what}"
    return f"k_scale_search_pair {what}" if len(modes) > 1 else f"k_scale_search {what}"


def centre_lo(cfg, label: str) -> int:
    """Offset of the exhaustive search's first 16-code block: the fused window's lo, else -8."""
    modes = label_modes(cfg, label)
    win = [m for m in modes if not m.exhaustive]
    return win[0].lo if len(modes) > 1 and win else -8


def pair_label(modes) -> str:
    return "search:" + "+".join(m.label for m in modes)


def base_label(label: str) -> str:
    """A call label without its matrix prefix ("mlp70b_up/search:..." -> "search:...")."""
    return label.split("/", 1)[1] if "/" in label else label


def label_modes(cfg, label: str):
    """The modes a search label covers (one mode's "search:A", or the paired "search:A+B")."""
    label = base_label(label)
    one = [m for m in cfg.modes if label == f"search:{m.label}"]
    if one:
        return one
    pair = paired_modes(cfg)
    return pair if pair is not None and label == pair_label(pair) else []


def search_work(cfg, label: str, scored=None):
    """(flops, lane-operations) of a search call. A windowed mode scores every candidate of its
    window for every weight, by the method's definition. The exhaustive mode skips the codes
    that a lower bound proves to lose, so its work is the number of (group, code) candidates it
    scores on the call's inputs (`scored`, from nvfp4_scale_search_scored), times 16 elements;
    a 16-code window fused with it is its first block, so it adds nothing."""
    modes = label_modes(cfg, label)
    flops = ops = 0
    exh = [m for m in modes if m.exhaustive]
    for m in modes:
        if m.exhaustive:
            n_ec = scored * 16
        elif exh:
            continue
        else:
            n_ec = cfg.n_weights * n_candidates(m)
        flops += n_ec * FLOPS_PER_ELEM_CAND[m.objective]
        ops += n_ec * OPS_PER_ELEM_CAND[m.objective]
    return flops, ops


def algorithmic_bytes(cfg, label: str) -> int:
    """Bytes one call must move by the definition: inputs read once, outputs written once."""
    label = base_label(label)
    n_w = cfg.n_weights
    wb = 2 if is_bf16(cfg) else 4
    T = cfg.chunk_tokens or cfg.tokens
    if label == "h_finalize":
        return cfg.batch * cfg.inp * 12
    if label == "h_reduce":
        return T * cfg.inp * 2 + (0 if cfg.chunk_tokens else cfg.batch * cfg.inp * 12)
    if label == "h_reduce_chunks":
        return cfg.tokens * cfg.inp * 2 + cfg.inp * 12
    if label == "global_scale":
        return n_w * wb + 4 * cfg.batch
    if label == "h_reduce+global_scale":
        return T * cfg.inp * 2 + cfg.inp * 12 + n_w * wb + 4
    modes = label_modes(cfg, label)
    nb = n_w * wb + len(modes) * (n_w // 2 + n_w // 16)
    if any(m.objective == "wmse" for m in modes):
        nb += cfg.batch * cfg.inp * 4
    if any(m.proposal for m in modes):
        nb += 2 * (n_w // 16)      # proposal and incoming code per group
    return nb


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


class Layer:
    """One input set of one matrix, resident on the GPU, plus its output buffers."""

    def __init__(self, cfg, k: int, dev):
        import torch

        from block_scale_search_amd import workloads
        cfg_k = type(cfg)(**{**cfg.__dict__, "seed": cfg.seed + 100 * k})
        self.cfg = cfg
        self.W = workloads.make_weights(cfg_k, dev)
        sigma = workloads.make_sigma(cfg_k, dev)
        self.chunks, self.seg = [], None
        for c in range(workloads.n_chunks(cfg)):
            X, offs = workloads.make_activation_chunk(cfg_k, sigma, c, dev)
            self.chunks.append(X)
            if offs is not None:
                self.seg = torch.from_numpy(offs).to(dev)
        n, E = cfg.inp, cfg.batch
        self.h_acc = torch.zeros((E, n) if E > 1 else (n,), dtype=torch.float64, device=dev)
        self.h = torch.empty((E, n) if E > 1 else (n,), dtype=torch.float32, device=dev)
        self.S = torch.empty(E, dtype=torch.float32, device=dev)
        G = cfg.batch * cfg.out * (n // 16)
        self.scales = [torch.empty(G, dtype=torch.uint8, device=dev) for _ in cfg.modes]
        self.packed = [torch.empty(G * 8, dtype=torch.uint8, device=dev) for _ in cfg.modes]


class Kind:
    """One matrix shape of the workload: its rotated input sets, workspaces and the calls of one
    layer."""

    def __init__(self, cfg, n_sets: int, dev, prefix: str, separate_stats: bool,
                 separate_searches: bool, h_per_chunk: bool):
        import torch

        from block_scale_search_amd import nvfp4, workloads
        self.nv, self.cfg, self.prefix = nvfp4, cfg, prefix
        self.separate_stats, self.separate_searches = separate_stats, separate_searches
        self.h_per_chunk = h_per_chunk
        self.sets = [Layer(cfg, k, dev) for k in range(n_sets)]
        T = cfg.chunk_tokens or cfg.tokens
        E = cfg.batch
        ws = nvfp4.nvfp4_diag_hessian_workspace_size(T, cfg.inp, E)
        if len(self.sets[0].chunks) > 1:
            ws = max(ws, nvfp4.nvfp4_diag_hessian_chunks_workspace_size(
                [X.shape[0] for X in self.sets[0].chunks], cfg.inp))
        self.ws_h = torch.zeros(max(16, ws), dtype=torch.uint8, device=dev)
        self.ws_s = torch.zeros(max(16, nvfp4.nvfp4_global_scale_workspace_size(E, cfg.out,
                                                                                 cfg.inp)),
                                dtype=torch.uint8, device=dev)
        self.ws_ls = torch.zeros(max(16, nvfp4.nvfp4_layer_statistics_workspace_size(
            T, cfg.inp, cfg.out)), dtype=torch.uint8, device=dev)
        self.rule = nvfp4.GS_AMAX_256 if cfg.gs_rule == "amax256" else nvfp4.GS_AMAX_448
        if any(m.proposal for m in cfg.modes):
            # proposal and incoming codes, made once outside the timed steps: the incoming code
            # is the max-abs base code, the proposal the base code moved by a seeded offset
            for s in self.sets:
                S = nvfp4.global_scale(s.W, self.rule)
                base = nvfp4.scale_search(s.W, None, S, nvfp4.MSE, 0, 0, with_stats=False)["scales"]
                off = workloads.proposal_offsets(cfg, base.shape, dev)
                s.center = (base.to(torch.int32) + off).clamp(1, 126).to(torch.uint8).contiguous()
                s.incoming = base.contiguous()
            torch.cuda.synchronize()

    def fused_stats(self, s) -> bool:
        return s.seg is None and len(s.chunks) == 1 and not self.separate_stats

    def h_calls(self, s, stream=None):
        """The calls that produce h (no global scale), as the step makes them; for a layer whose
        step computes h and S in one call, the plain h-reduce call instead."""
        nv, cfg = self.nv, self.cfg
        n = cfg.inp
        out = []
        deferred = len(s.chunks) > 1 and s.seg is None
        if deferred and not self.h_per_chunk:
            # every resident token chunk of the set in one partial launch and one finalize
            return [("h_reduce_chunks", nv.nvfp4_diag_hessian_chunks(
                s.chunks, n, n, s.h_acc, s.h, False, self.ws_h, stream=stream, prepare=True))]
        for ci, X in enumerate(s.chunks):
            T = X.shape[0]
            if s.seg is not None:
                out.append(("h_reduce", nv.nvfp4_diag_hessian_batched(
                    X, s.seg, cfg.batch, T, n, n, s.h_acc, s.h, ci > 0, self.ws_h, stream=stream,
                    prepare=True)))
            elif deferred:
                # token chunks of one calibration set: row-group sums accumulate in the
                # workspace, one finalize after the last chunk
                out.append(("h_reduce", nv.nvfp4_diag_hessian(
                    X, T, n, n, None, None, ci > 0, self.ws_h, stream=stream, prepare=True)))
            else:
                out.append(("h_reduce", nv.nvfp4_diag_hessian(
                    X, T, n, n, s.h_acc, s.h, ci > 0, self.ws_h, stream=stream, prepare=True)))
        if deferred:
            out.append(("h_finalize", nv.nvfp4_diag_hessian_finalize(
                s.chunks[0].dtype, s.chunks[0].shape[0], n, s.h_acc, s.h, False, self.ws_h,
                stream=stream, prepare=True)))
        return out

    def calls(self, s, stage=None, search=None):
        """One layer as (label, call, role) triples in issue order; each call is a prepared C-ABI
        invocation (arguments marshalled once). Role "stage": produces h and S (on the stage
        stream under the pipeline); role "main": the searches (on `search`, default the current
        stream)."""
        nv, cfg = self.nv, self.cfg
        b, o, n = cfg.batch, cfg.out, cfg.inp
        ldw, sw = n, o * n
        out = []
        if self.fused_stats(s):
            # one matrix, one token chunk: h and S in one call (two launches)
            X = s.chunks[0]
            out.append(("h_reduce+global_scale", nv.nvfp4_layer_statistics(
                X, X.shape[0], n, n, s.h_acc, s.h, False, s.W, o, ldw, self.rule, s.S,
                self.ws_ls, stream=stage, prepare=True), "stage"))
        else:
            out += [(lab, f, "stage") for lab, f in self.h_calls(s, stage)]
            out.append(("global_scale", nv.nvfp4_global_scale(
                s.W, b, o, n, ldw, sw, self.rule, s.S, self.ws_s, stream=stage, prepare=True),
                "stage"))
        pair = None if self.separate_searches else paired_modes(cfg)
        if pair is not None:
            # two rules in one call and one launch: two windows read each group once for both,
            # or a 16-code window is the exhaustive search's first block
            idx = [cfg.modes.index(m) for m in pair]
            wm_any = any(m.objective == "wmse" for m in pair)
            rules = [dict(objective=nv.WMSE if m.objective == "wmse" else nv.MSE, lo=m.lo,
                          hi=m.hi, exhaustive=m.exhaustive, scales=s.scales[i],
                          packed=s.packed[i])
                     for m, i in zip(pair, idx)]
            out.append((pair_label(pair), nv.nvfp4_scale_search_rules(
                s.W, b, o, n, ldw, sw, 16, s.h if wm_any else None, n if wm_any else 0, s.S,
                rules, stream=search, prepare=True), "main"))
        for mi, m in enumerate(cfg.modes):
            wm = m.objective == "wmse"
            if pair is not None and m in pair:
                continue
            if m.proposal:
                out.append((f"search:{m.label}", nv.nvfp4_scale_search_proposal(
                    s.W, b, o, n, ldw, sw, 16, s.h if wm else None, n if wm else 0,
                    nv.WMSE if wm else nv.MSE, m.lo, m.hi, s.center, s.incoming, s.S,
                    s.scales[mi], s.packed[mi], stream=search, prepare=True), "main"))
                continue
            out.append((f"search:{m.label}", nv.nvfp4_scale_search(
                s.W, b, o, n, ldw, sw, 16, s.h if wm else None, n if wm else 0,
                nv.WMSE if wm else nv.MSE, m.lo, m.hi, m.exhaustive, s.S, s.scales[mi],
                s.packed[mi], stream=search, prepare=True), "main"))
        return [(self.prefix + lab, f, role) for lab, f, role in out]


def cpu_baseline(kinds, threads: int):
    """The oracle, as it stands, on a bounded sample of each matrix's first input set (the GPU's
    own inputs, copied to the host), projected to the whole step, plus the parity of that
    sample with the GPU's outputs of the timed steps.

    Sample per matrix: up to 2^24 weights (whole rows, or whole experts of a batch) and the
    tokens of the first chunk (or of the sampled experts). Passes are repeated until at least
    10 s of wall time. Projection: the h time scales with the step's tokens over the sampled
    tokens, the global-scale and search time with the step's weights over the sampled weights.
    S is a whole-tensor quantity, and h sums every token chunk: the searches take the oracle's
    S of the whole matrix and its h over every chunk, both computed once outside the timing.
    """
    import numpy as np

    import oracle

    budget = 1 << 24
    samples = []
    for kd in kinds:
        cfg, layer = kd.cfg, kd.sets[0]
        rule = oracle.GS_AMAX_256 if cfg.gs_rule == "amax256" else oracle.GS_AMAX_448
        center = incoming = None
        if cfg.batch == 1:
            R = max(1, min(cfg.out, budget // cfg.inp))
            Ws = [host_array(layer.W[:R])]
            if hasattr(layer, "center"):
                center = layer.center[:R].cpu().numpy()
                incoming = layer.incoming[:R].cpu().numpy()
            X0 = [host_array(layer.chunks[0])]
            # h over every chunk and S of the whole matrix, untimed
            acc = None
            for X in layer.chunks:
                acc, h_full = oracle.diag_hessian(host_array(X), acc, threads=threads)
            h_all = [h_full]
            S_all = [oracle.global_scale(host_array(layer.W), rule)]
            w_frac = cfg.out / R
            tok_sample = layer.chunks[0].shape[0]
            desc = f"{R} of {cfg.out} rows"
        else:
            E = max(1, min(cfg.batch, budget // (cfg.out * cfg.inp)))
            Ws = [host_array(layer.W[e]) for e in range(E)]
            seg = layer.seg.cpu().numpy()
            X0 = [host_array(layer.chunks[0][int(seg[e]):int(seg[e + 1])]) for e in range(E)]
            h_all = [oracle.diag_hessian(x, None, threads=threads)[1] for x in X0]
            S_all = [oracle.global_scale(w, rule) for w in Ws]
            w_frac = cfg.batch / E
            tok_sample = int(seg[E])
            desc = f"{E} of {cfg.batch} experts"
        samples.append(dict(kd=kd, rule=rule, Ws=Ws, X0=X0, h_all=h_all, S_all=S_all,
                            center=center, incoming=incoming, w_frac=w_frac,
                            tok_frac=cfg.tokens / max(1, tok_sample), tok_sample=tok_sample,
                            desc=desc, t_h=0.0, t_s=0.0, first=[]))

    passes = 0
    t0 = time.perf_counter()
    while True:
        for sm in samples:
            cfg = sm["kd"].cfg
            for i, (W, X) in enumerate(zip(sm["Ws"], sm["X0"])):
                a = time.perf_counter()
                oracle.diag_hessian(X, None, threads=threads)
                b = time.perf_counter()
                oracle.global_scale(W, sm["rule"])
                S_o, h = sm["S_all"][i], sm["h_all"][i]
                res = []
                for m in cfg.modes:
                    wm = m.objective == "wmse"
                    if m.proposal:
                        res.append(oracle.scale_search_proposal(
                            W, h if wm else None, oracle.WMSE if wm else oracle.MSE, m.lo, m.hi,
                            sm["center"], sm["incoming"], S_o, threads=threads))
                    else:
                        res.append(oracle.scale_search(
                            W, h if wm else None, oracle.WMSE if wm else oracle.MSE, m.lo,
                            m.hi, m.exhaustive, S_o, threads=threads))
                c = time.perf_counter()
                sm["t_h"] += b - a
                sm["t_s"] += c - b
                if passes == 0:
                    sm["first"].append([r_["scales"] for r_ in res])
        passes += 1
        if time.perf_counter() - t0 >= 10.0:
            break
    step_s = sum(sm["t_h"] * sm["tok_frac"] + sm["t_s"] * sm["w_frac"] for sm in samples) / passes
    layer_weights = sum(sm["kd"].cfg.n_weights for sm in samples)
    parity = {sm["kd"].cfg.name: parity_on_sample(sm) for sm in samples}
    return {"value": layer_weights / step_s, "unit": "weights/s", "cores": threads,
            "kind": "oracle",
            "sample": "; ".join(
                f"{sm['kd'].cfg.name}: first input set, {sm['desc']} and {sm['tok_sample']} of "
                f"{sm['kd'].cfg.tokens} tokens, h + global scale + "
                f"{' + '.join(m.label for m in sm['kd'].cfg.modes)}, projected (h time x "
                f"{sm['tok_frac']:.3g}, search time x {sm['w_frac']:.3g})" for sm in samples)
            + f"; {passes} passes in {time.perf_counter() - t0:.1f} s on {threads} threads",
            "parity_on_sample": parity if len(parity) > 1 else next(iter(parity.values()))}


def parity_on_sample(sm):
    """The GPU's own outputs of the timed steps against the oracle's first pass on the sampled
    rows or experts: h over every token chunk (largest relative difference), S (equal or not),
    and for each mode the number of groups whose scale byte differs. The GPU's searches used the
    GPU's h and the oracle's its own, so a WMSE mode's count includes any flip that h's rounding
    causes (none when every h element agrees)."""
    import numpy as np
    cfg, layer = sm["kd"].cfg, sm["kd"].sets[0]
    hg = layer.h.cpu().numpy().reshape(cfg.batch, cfg.inp)
    Sg = layer.S.cpu().numpy().reshape(-1)
    gpr = cfg.inp // 16
    sc = [x.cpu().numpy().reshape(cfg.batch, cfg.out, gpr) for x in layer.scales]
    h_rel, s_eq, mism, groups = 0.0, True, [0] * len(cfg.modes), 0
    for e, (h_o, S_o, scales_o) in enumerate(zip(sm["h_all"], sm["S_all"], sm["first"])):
        ho = np.asarray(h_o, dtype=np.float64).reshape(-1)
        d = np.abs(hg[e].astype(np.float64) - ho) / np.maximum(np.abs(ho), 1e-30)
        h_rel = max(h_rel, float(d.max()))
        s_eq = s_eq and bool(np.float32(S_o) == Sg[e])
        for mi, so in enumerate(scales_o):
            so = np.asarray(so).reshape(-1, gpr)
            mism[mi] += int((sc[mi][e][:so.shape[0]] != so).sum())
        groups += np.asarray(scales_o[0]).size
    return {"groups": groups, "h_chunks": len(layer.chunks), "h_max_rel_diff": h_rel,
            "S_equal": s_eq,
            "scale_mismatches": {m.label: mism[i] for i, m in enumerate(cfg.modes)}}


def cpu_single_core(cfg, layer):
    """The oracle on one host thread, for the single-matrix workloads up to 2^26 weights: one pass
    over about 2^20 weights (whole rows) and at most 2048 tokens, projected to the whole step by
    the weight and token ratios."""
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
    return {"value": cfg.n_weights / step_s, "unit": "weights/s", "cores": 1,
            "sample": f"{R} of {cfg.out} rows and {X.shape[0]} of {cfg.tokens} tokens, one pass, "
                      f"projected (h time x {tok_frac:.3g}, search time x {w_frac:.3g})"}


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
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="mlp70b (both 70B MLP matrices per step), or one of tiny, attn8b, "
                         "down8b, moe, mlp70b_up, mlp70b_down, mlp70b_up_proposal")
    ap.add_argument("--sets", type=int, default=0, help="input sets rotated (0 = enough for >1 GB)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--separate-stats", action="store_true",
                    help="h and S as two calls (nvfp4_diag_hessian, nvfp4_global_scale) instead "
                         "of nvfp4_layer_statistics on one-chunk workloads")
    ap.add_argument("--separate-searches", action="store_true",
                    help="one nvfp4_scale_search call per mode instead of one "
                         "nvfp4_scale_search_rules call for a pair of windowed modes")
    ap.add_argument("--h-per-chunk", action="store_true",
                    help="chunked X: one deferred nvfp4_diag_hessian call per token chunk and one "
                         "finalize, instead of one nvfp4_diag_hessian_chunks call over all of a "
                         "set's resident chunks")
    ap.add_argument("--schedule", default="pipeline", choices=("pipeline", "sequential"),
                    help="pipeline: the next layer's h and S calls run on a second stream while "
                         "this layer's searches run; sequential: every call on one stream, in "
                         "order")
    ap.add_argument("--search-streams", type=int, default=1, choices=(1, 2),
                    help="layer pipeline: consecutive layers' searches on 1 stream, or on 2 "
                         "alternating streams so that one layer's search starts while the "
                         "previous one's last workgroups finish")
    ap.add_argument("--events-every", type=int, default=8,
                    help="record per-call HIP events on every Nth timed step (1 = all)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--activations", action="store_true",
                    help="also time on-line activation quantisation (dynamic S + MSE [-3,7]) of "
                         "the first token chunk and of a 16-token decode batch, outside the step")
    ap.add_argument("--gptq", action="store_true",
                    help="also time GPTQ with the window search as local quantiser on the first "
                         "matrix (U from X^T X of the first token chunk, 1%% damping), outside "
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
    if args.workload not in workloads.CONFIGS and args.workload not in workloads.GROUPS:
        ap.error(f"unknown workload {args.workload}")
    cfgs = workloads.workload_configs(args.workload)
    group = len(cfgs) > 1
    dev = torch.device("cuda:0")
    per_set = sum(c.n_weights * (2 if is_bf16(c) else 4) + c.tokens * c.inp * 2 for c in cfgs)
    # enough sets for more than 1 GiB of inputs (past the 256 MB MALL), at most 8; the layer
    # pipeline needs at least two
    n_sets = args.sets or max(2 if args.schedule == "pipeline" else 1,
                              min(8, -(-(1 << 30) // per_set)))
    print(f"# workload {args.workload}: {'; '.join(c.description for c in cfgs)}; {n_sets} "
          f"input set(s)", file=sys.stderr, flush=True)
    kinds = [Kind(c, n_sets, dev, f"{c.name}/" if group else "", args.separate_stats,
                  args.separate_searches, args.h_per_chunk) for c in cfgs]
    torch.cuda.synchronize()

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    main_st = torch.cuda.current_stream()
    pipelined = args.schedule == "pipeline" and (n_sets >= 2 or len(kinds) >= 2)
    schedule = "pipeline" if pipelined else "sequential"
    stage = torch.cuda.Stream() if pipelined else None
    R = len(kinds)
    # layer j of the rotation: matrix kind j % R, input set (j // R) % n_sets; step i = layers
    # i R .. i R + R - 1. With two search streams, layer j's searches run on stream
    # (j mod R n_sets) mod 2, which alternates between consecutive layers when R n_sets is even.
    search_sts = [main_st] + ([torch.cuda.Stream()] if pipelined and args.search_streams == 2
                              else [])

    def search_stream(r, k):
        return search_sts[(r + R * k) % len(search_sts)]
    layer_calls = [[kd.calls(s, stage, search_stream(r, k)) for k, s in enumerate(kd.sets)]
                   for r, kd in enumerate(kinds)]
    step_labels = [lab for r in range(R) for lab, _, _ in layer_calls[r][0]]

    def calls_of(j):
        return layer_calls[j % R][(j // R) % n_sets]

    def timed_call(lab, f, st, row):
        if row is None:
            f()
            return
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        f()
        e1.record(st)
        row.append((lab, e0, e1))

    ev_stage = [[torch.cuda.Event() for _ in range(n_sets)] for _ in range(R)]
    ev_done = [[torch.cuda.Event() for _ in range(n_sets)] for _ in range(R)]

    def run_layers(first_step, n_steps, rows=None):
        """Steps first_step .. first_step + n_steps - 1. rows (a dict) receives each timed step's
        (label, start, end) event triples."""
        def row_of(j):
            i = j // R
            if rows is None or (i - first_step) % args.events_every:
                return None
            return rows.setdefault(i, [])

        j0, j1 = first_step * R, (first_step + n_steps) * R
        if j1 <= j0:
            return
        if not pipelined:
            for j in range(j0, j1):
                for lab, f, _ in calls_of(j):
                    timed_call(lab, f, main_st, row_of(j))
            return

        def issue_stage(j):
            r, k = j % R, (j // R) % n_sets
            if j - j0 >= R * n_sets:
                stage.wait_event(ev_done[r][k])       # the set's previous searches are done
            for lab, f, role in calls_of(j):
                if role == "stage":
                    timed_call(lab, f, stage, row_of(j))
            ev_stage[r][k].record(stage)

        stage.wait_stream(main_st)
        for st in search_sts[1:]:
            st.wait_stream(main_st)
        issue_stage(j0)
        for j in range(j0, j1):
            r, k = j % R, (j // R) % n_sets
            if j + 1 < j1:
                issue_stage(j + 1)
            st = search_stream(r, k)
            st.wait_event(ev_stage[r][k])
            for lab, f, role in calls_of(j):
                if role != "stage":
                    timed_call(lab, f, st, row_of(j))
            ev_done[r][k].record(st)
        main_st.wait_stream(stage)
        for st in search_sts[1:]:
            main_st.wait_stream(st)

    run_layers(0, args.warmup)
    torch.cuda.synchronize()

    rows = {}
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(main_st)
    run_layers(args.warmup, args.steps, rows)
    t_end.record(main_st)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps

    p0 = torch.cuda.Event(enable_timing=True)
    p1 = torch.cuda.Event(enable_timing=True)

    def back_to_back(fs, reps):
        """Average us per call of fs[i % len(fs)] over reps calls on the main stream."""
        for f in fs:
            f()
        torch.cuda.synchronize()
        p0.record(main_st)
        for i in range(reps):
            fs[i % len(fs)]()
        p1.record(main_st)
        torch.cuda.synchronize()
        return p0.elapsed_time(p1) * 1e3 / reps

    nv = kinds[0].nv
    kind_of = {}
    for kd in kinds:
        for lab, _, _ in layer_calls[kinds.index(kd)][0]:
            kind_of[lab] = kd
    # the work of each search call with an exhaustive mode: the candidates it scores on each
    # input set (every set's h and S made again first, outside the timing; same values)
    alone_calls = [[kd.calls(s) for s in kd.sets] for kd in kinds]   # all on the main stream
    for r in range(R):
        for calls in alone_calls[r]:
            for _, f, role in calls:
                if role == "stage":
                    f()
    torch.cuda.synchronize()
    scored = {}
    for lab in dict.fromkeys(l for l in step_labels if base_label(l).startswith("search")):
        kd = kind_of[lab]
        e = next((m for m in label_modes(kd.cfg, lab) if m.exhaustive), None)
        if e is None:
            continue
        wm = e.objective == "wmse"
        counts = [nv.scale_search_scored(s.W, s.h if wm else None, s.S,
                                         nv.WMSE if wm else nv.MSE, centre_lo(kd.cfg, lab))
                  for s in kd.sets]
        scored[lab] = sum(counts) / len(counts)
    kernels = {}
    per_label = {}
    for i in sorted(rows):
        for lab, e0, e1 in rows[i]:
            per_label.setdefault(lab, []).append(e0.elapsed_time(e1) * 1e3)  # us
    steps_timed = len(rows)
    for lab, us in per_label.items():
        cfg = kind_of[lab].cfg
        per_step = step_labels.count(lab)
        us_avg = sum(us) / len(us)
        nb = algorithmic_bytes(cfg, lab)
        k = {"avg_us": round(us_avg, 3), "calls_per_step": per_step,
             "alg_bytes": nb, "GB/s": round(nb / us_avg / 1e3, 1),
             "frac_hbm": round(nb / us_avg / 1e3 / HBM_PEAK_GBS, 4)}
        if base_label(lab).startswith("search"):
            k["weights/s"] = cfg.n_weights / (us_avg * 1e-6)
            nf, no = search_work(cfg, lab, scored.get(lab))
            k["TFLOP/s"] = round(nf / us_avg / 1e6, 2)
            k["frac_157.3_TFLOP/s"] = round(nf / us_avg / 1e6 / VALU_PUBLISHED_TFLOPS, 4)
            k["frac_valu_issue"] = round(no / us_avg / 1e6 / VALU_ISSUE_TOPS, 4)
            if lab in scored:
                groups = cfg.n_weights // 16
                k["scored_codes_per_group"] = round(scored[lab] / groups, 3)
                # every one of the 126 codes counted, as an unpruned search would score them
                e = next(m for m in label_modes(cfg, lab) if m.exhaustive)
                k["TFLOP/s_126_equivalent"] = round(
                    groups * 126 * 16 * FLOPS_PER_ELEM_CAND[e.objective] / us_avg / 1e6, 2)
        kernels[lab] = k

    # the h stage of each matrix in the step: all chunk calls plus the finalize (or the one
    # call that computes h and S), over the bytes they must read
    for kd in kinds:
        cfg, p = kd.cfg, kd.prefix
        x_bytes = cfg.tokens * cfg.inp * 2
        if p + "h_reduce+global_scale" in kernels:
            kk = kernels[p + "h_reduce+global_scale"]
            kernels[p + "h+S stage (one call, X and W bytes)"] = {
                "us_per_step": kk["avg_us"], "bytes": kk["alg_bytes"], "GB/s": kk["GB/s"],
                "frac_hbm": kk["frac_hbm"]}
        else:
            lab = p + ("h_reduce_chunks" if p + "h_reduce_chunks" in kernels else "h_reduce")
            h_us = kernels[lab]["avg_us"] * kernels[lab]["calls_per_step"]
            if p + "h_finalize" in kernels:
                h_us += kernels[p + "h_finalize"]["avg_us"]
            gbs = x_bytes / h_us / 1e3
            kernels[p + "h stage in the step (all chunks + finalize)"] = {
                "us_per_step": round(h_us, 2), "x_bytes": x_bytes, "GB/s": round(gbs, 1),
                "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}

    # outside the step, back to back over the input sets: each matrix's h stage alone (the
    # plain h-reduce call where the step fuses h and S), the pack at given scales, and each
    # search call
    h_alone = {}
    for kd in kinds:
        cfg, p = kd.cfg, kd.prefix
        per_layer = [kd.h_calls(s) for s in kd.sets]
        n_calls = len(per_layer[0])
        fs = [f for calls in per_layer for _, f in calls]
        us = back_to_back(fs, len(fs) * max(2, -(-20 // len(fs)))) * n_calls
        x_bytes = cfg.tokens * cfg.inp * 2
        h_alone[cfg.name] = {"us": round(us, 2), "x_bytes": x_bytes,
                             "calls": [lab for lab, _ in per_layer[0]][:2] +
                                      ([f"... {n_calls} calls"] if n_calls > 2 else []),
                             "GB/s": round(x_bytes / us / 1e3, 1),
                             "frac_hbm": round(x_bytes / us / 1e3 / HBM_PEAK_GBS, 4)}
        packs = [nv.nvfp4_pack(s.W, cfg.batch, cfg.out, cfg.inp, cfg.inp, cfg.out * cfg.inp,
                               s.scales[-1], s.S, s.packed[-1], prepare=True) for s in kd.sets]
        pack_us = back_to_back(packs, 50 * len(packs))
        wb = 2 if is_bf16(cfg) else 4
        pack_bytes = cfg.n_weights * wb + cfg.n_weights // 2 + cfg.n_weights // 16
        kernels[p + "pack (outside the step)"] = {
            "avg_us": round(pack_us, 3), "calls_per_step": 0, "alg_bytes": pack_bytes,
            "GB/s": round(pack_bytes / pack_us / 1e3, 1),
            "frac_hbm": round(pack_bytes / pack_us / 1e3 / HBM_PEAK_GBS, 4)}
    search_alone = {}
    for lab in dict.fromkeys(l for l in step_labels if base_label(l).startswith("search")):
        fs = [f for r in range(R) for calls in alone_calls[r] for l, f, _ in calls if l == lab]
        search_alone[lab] = back_to_back(fs, max(4, 3 * len(fs)))
        kernels[lab]["alone_us"] = round(search_alone[lab], 3)

    # roofline: the fixed-work search (same mode over every matrix of the step) with the
    # largest share of the step
    groups = {}
    for lab in dict.fromkeys(l for l in step_labels if base_label(l).startswith("search")):
        g = groups.setdefault(base_label(lab), {"labels": [], "us": 0.0, "flops": 0, "ops": 0,
                                                "bytes": 0, "launches": 0, "alone_us": 0.0})
        cfg = kind_of[lab].cfg
        nf, no = search_work(cfg, lab, scored.get(lab))
        n_per = step_labels.count(lab)
        g["labels"].append(lab)
        g["us"] += kernels[lab]["avg_us"] * n_per
        g["flops"] += nf * n_per
        g["ops"] += no * n_per
        g["bytes"] += algorithmic_bytes(cfg, lab) * n_per
        g["launches"] += n_per
        g["alone_us"] += search_alone[lab] * n_per
    # the search call (same mode or modes over every matrix of the step) with the largest share
    # of the step
    dom = max(groups, key=lambda k: groups[k]["us"])
    g = groups[dom]
    us_launch = g["us"] / g["launches"]
    achieved = g["flops"] / g["us"] / 1e6
    dom_kd = kind_of[g["labels"][0]]
    pruned = any(m.exhaustive for m in label_modes(dom_kd.cfg, g["labels"][0]))
    roofline = {
        "bound": "alu", "kernel": kernel_name(dom_kd.cfg, g["labels"][0]),
        "achieved": round(achieved, 2), "peak": VALU_PUBLISHED_TFLOPS, "unit": "TFLOP/s",
        "frac": round(achieved / VALU_PUBLISHED_TFLOPS, 4),
        "traffic": read_traffic(args.workload, dom),
        "alg_flops_per_launch": int(round(g["flops"] / g["launches"])),
        "avg_launch_us": round(us_launch, 3), "launches_per_step": g["launches"],
        "flops_per_element_candidate": FLOPS_PER_ELEM_CAND,
        "flops_counted": ("element-candidates the exhaustive search scores (its first block of "
                          "16 codes, which is the fused window, plus every block of 4 that its "
                          "exact lower bounds keep; nvfp4_scale_search_scored on the same "
                          "inputs), x flops per element-candidate" if pruned else
                          "every candidate of the window for every weight, x flops per "
                          "element-candidate"),
        "share_of_step": round(g["us"] / (ms_per_step * 1e3), 4),
        "lane_issue": {"achieved": round(g["ops"] / g["us"] / 1e6, 2), "peak": VALU_ISSUE_TOPS,
                       "unit": "T lane-operations/s",
                       "frac": round(g["ops"] / g["us"] / 1e6 / VALU_ISSUE_TOPS, 4),
                       "note": "each lane-operation is one fp32 VALU operation (rounding "
                               "included, fma = 1); the build emits no packed fp32, so this "
                               "issue rate, not 157.3 TFLOP/s, is the kernel's ceiling"},
        "hbm": {"alg_bytes_per_launch": g["bytes"] // g["launches"],
                "GB/s": round(g["bytes"] / g["us"] / 1e3, 1),
                "frac": round(g["bytes"] / g["us"] / 1e3 / HBM_PEAK_GBS, 4)},
        "alone": {"avg_launch_us": round(g["alone_us"] / g["launches"], 3),
                  "achieved": round(g["flops"] / g["alone_us"] / 1e6, 2),
                  "frac": round(g["flops"] / g["alone_us"] / 1e6 / VALU_PUBLISHED_TFLOPS, 4),
                  "note": "the same calls back to back outside the timed steps; in the steps "
                          "they share the compute units with the next layer's h and S"},
    }
    if pruned:
        groups_per_launch = sum(kind_of[l].cfg.n_weights // 16 * step_labels.count(l)
                                for l in g["labels"]) / g["launches"]
        e = next(m for m in label_modes(dom_kd.cfg, g["labels"][0]) if m.exhaustive)
        eq = groups_per_launch * 126 * 16 * FLOPS_PER_ELEM_CAND[e.objective]
        roofline["scored_codes_per_group"] = round(
            sum(scored[l] * step_labels.count(l) for l in g["labels"]) / g["launches"]
            / groups_per_launch, 3)
        roofline["TFLOP/s_126_equivalent"] = round(eq / us_launch / 1e6, 2)
    others = {k: v for k, v in groups.items() if k != dom}
    if others:
        roofline["other_searches"] = {
            k: {"us_per_step": round(v["us"], 2),
                "share_of_step": round(v["us"] / (ms_per_step * 1e3), 4),
                "TFLOP/s": round(v["flops"] / v["us"] / 1e6, 2),
                "frac": round(v["flops"] / v["us"] / 1e6 / VALU_PUBLISHED_TFLOPS, 4)}
            for k, v in others.items()}

    extras = run_extras(args, kinds[0], dev, p0, p1, main_st, back_to_back)

    cpu = None
    if not args.no_cpu:
        threads = min(16, len(os.sched_getaffinity(0)))
        cpu = cpu_baseline(kinds, threads)
        if not group:
            one = cpu_single_core(kinds[0].cfg, kinds[0].sets[0])
            if one is not None:
                cpu["single_core"] = one

    layer_weights = sum(c.n_weights for c in cfgs)
    searches = sum(c.n_weights * len(c.modes) for c in cfgs)
    h_stage = {}
    for kd in kinds:
        p = kd.prefix
        k = kernels.get(p + "h stage in the step (all chunks + finalize)") or \
            kernels.get(p + "h+S stage (one call, X and W bytes)")
        h_stage[kd.cfg.name] = k["GB/s"]
    description = {
        "mlp70b": "70B-shaped MLP pair: W 28672x8192 and 8192x28672 bf16 (student-t df=5), X "
                  "65536x8192 and 65536x28672 bf16 streamed in 8192-token chunks; WMSE [-9,6] "
                  "and exhaustive 126-code mode on each"}.get(args.workload, cfgs[0].description)
    line = {
        "metric": METRIC,
        "value": layer_weights / (ms_per_step * 1e-3),
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
        "config": {"workload": description, "name": args.workload,
                   "matrices": [f"{c.name} {c.out}x{c.inp}" + (f" x{c.batch}" if c.batch > 1 else "")
                                for c in cfgs],
                   "modes": {c.name: [m.label for m in c.modes] for c in cfgs},
                   "tokens": {c.name: c.tokens for c in cfgs},
                   "chunk_tokens": {c.name: c.chunk_tokens or c.tokens for c in cfgs},
                   "global_scale": {c.name: c.gs_rule for c in cfgs},
                   "layer_weights_per_step": layer_weights,
                   "weight_searches_per_step": searches,
                   "input_sets_rotated": n_sets, "schedule": schedule,
                   "search_streams": len(search_sts),
                   "timed_steps_with_events": steps_timed},
        "weight_searches_per_s": searches / (ms_per_step * 1e-3),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "h_reduce_GB/s": h_stage if group else next(iter(h_stage.values())),
        "h_reduce_alone": h_alone,
        **extras,
    }
    print(json.dumps(line), flush=True)


def run_extras(args, kd, dev, p0, p1, main_st, back_to_back):
    """Optional figures outside the step, on the workload's first matrix: the layer-output error
    (MFMA), on-line activation quantisation, GPTQ with the window search."""
    import torch
    nv, cfg = kd.nv, kd.cfg
    out = {}
    if args.output_error and cfg.batch == 1:
        T0 = kd.sets[0].chunks[0].shape[0]
        ws_oe = torch.empty(nv.nvfp4_output_error_workspace_size(T0, cfg.out, cfg.inp),
                            dtype=torch.uint8, device=dev)
        errs = [torch.empty(cfg.out, dtype=torch.float64, device=dev) for _ in kd.sets]
        calls_oe = [nv.nvfp4_output_error(s_.chunks[0], T0, cfg.inp, cfg.inp, s_.W, cfg.out,
                                          cfg.inp, s_.scales[-1], s_.packed[-1], s_.S, e_, False,
                                          ws_oe, prepare=True)
                    for s_, e_ in zip(kd.sets, errs)]
        oe_us = back_to_back(calls_oe, max(2 * len(calls_oe), 10))
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
            s_ = kd.sets[0]
            Xh, Wh = host_array(s_.chunks[0][:Ts]), host_array(s_.W)
            ph = host_array(s_.packed[-1]).reshape(cfg.out, cfg.inp // 2)
            sh = host_array(s_.scales[-1]).reshape(cfg.out, cfg.inp // 16)
            Sh = float(s_.S.item())
            t_cpu = cpu_time(lambda: oracle.output_error(Xh, Wh, ph, sh, Sh))
            oe["cpu_oracle"] = {"kind": "oracle", "us_projected": round(t_cpu * 1e6 * T0 / Ts, 1),
                                "sample": f"{Ts} of {T0} tokens, projected by the token ratio",
                                "cores": len(os.sched_getaffinity(0)),
                                "note": "binary64 numpy (its matmul uses the BLAS threads)"}
        out["output_error"] = oe

    if args.activations:
        acts = {}
        X0 = kd.sets[0].chunks[0]
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
            us1 = back_to_back([one], 200)
            us2 = back_to_back([lambda: (gs(), se())], 200)
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
        out["activations"] = acts

    if args.gptq and cfg.batch == 1:
        # the damped inverse-Hessian factor is the caller's preparation (binary64 Gram matrix,
        # inverse and Cholesky), outside the timing: only the library call is timed
        from block_scale_search_amd import workloads as workloads_mod
        s0 = kd.sets[0]
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
        g_us = back_to_back([call], 3)
        n_fma = cfg.out * cfg.inp * (cfg.inp - 1) / 2
        search_ops = cfg.out * cfg.inp * n_candidates(m) * OPS_PER_ELEM_CAND["wmse"]
        gq = {"ms": round(g_us / 1e3, 3), "mode": f"WMSE [{m.lo},{m.hi}]",
              "ordered_fmas": n_fma, "search_lane_ops": search_ops,
              "TOP/s": round((n_fma + search_ops) / g_us / 1e6, 2),
              "frac_valu_issue": round((n_fma + search_ops) / g_us / 1e6 / VALU_ISSUE_TOPS, 4),
              "weights/s": cfg.out * cfg.inp / (g_us * 1e-6),
              "note": "the library call only: the caller's Gram matrix, damping and "
                      "factorisation of U are outside the timing"}
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
        out["gptq"] = gq
    return out


if __name__ == "__main__":
    main()
