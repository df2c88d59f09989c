"""Seeded synthetic layer workloads (weights W and calibration activations X).

This module only draws random numbers: it holds none of the method's arithmetic, and both the
GPU library's callers and the CPU oracle's tests take their inputs from here.

The pages measure on trained checkpoints and on calibration sets that are not available here
(H-Scale: FineWeb calibration samples, 4,096 x 8,192 tokens; ScaleSweep: GSM8K train split;
Schur Replay: a 255-document set). Synthetic tensors of the layer shapes below stand in for them:

  tiny     W 256x256 fp32, 0.02*N(0,1), 0.5% entries x20;      X 512x256, channel std e^N(0,1)
  attn8b   W 4096x4096 bf16, 0.02*N(0,1), 0.1% entries x30;    X 8192x4096, channel std e^(1.5 N)
  down8b   W 4096x14336 bf16, 0.015*t(4);                      X 16384x14336, N(0,1), 1% chans x50
  moe      128 experts x W 768x2048 bf16, 0.02*N(0,1);         X 262144x2048 in 128 Zipf segments,
                                                               per-expert channel std e^N(0,1)
  mlp70b   W 28672x8192 and 8192x28672 bf16, 0.015*t(5);       X 65536x{8192, 28672}, std e^(1.5 N),
                                                               streamed in 8192-token chunks
  mlp70b_up_proposal  the 70B up/gate layer with proposal codes = base codes + U{-3..3}

Every tensor is drawn as float32 from a torch.Generator seeded per (config, stream) and then
rounded to bf16 (round-to-nearest-even) where the config says bf16. Student-t variates are
Z / sqrt(V / df) with V a sum of df squared normals. Outlier entries are chosen uniformly
without replacement. Zipf token counts are proportional to 1/rank over a seeded permutation of
the experts, rounded by largest remainder to the stated total with every count >= 1.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

# stream ids: one independent generator per (config seed, stream)
_W, _OUT, _SIGMA, _X, _ZIPF, _PROP = 1, 2, 3, 4, 5, 6


def _gen(seed: int, stream: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 64 + stream)
    return g


def normal_weights(out: int, inp: int, std: float, outlier_frac: float, outlier_mult: float,
                   seed: int, device="cpu", dtype=torch.bfloat16, batch: int | None = None):
    """std*N(0,1) weights; a fraction of entries (uniform, without replacement) multiplied."""
    shape = (out, inp) if batch is None else (batch, out, inp)
    g = _gen(seed, _W, device)
    w = torch.randn(shape, generator=g, device=device, dtype=torch.float32).mul_(std)
    n_out = int(round(outlier_frac * w.numel()))
    if n_out > 0:
        go = _gen(seed, _OUT, device)
        idx = torch.randperm(w.numel(), generator=go, device=device)[:n_out]
        w.view(-1)[idx] *= outlier_mult
    return w.to(dtype)


def student_t_weights(out: int, inp: int, df: int, scale: float, seed: int, device="cpu",
                      dtype=torch.bfloat16, row_chunk: int = 2048):
    """scale * t(df) weights, t = Z / sqrt(chi2_df / df) from df+1 normals per entry."""
    g = _gen(seed, _W, device)
    w = torch.empty((out, inp), device=device, dtype=dtype)
    for r0 in range(0, out, row_chunk):
        r1 = min(out, r0 + row_chunk)
        z = torch.randn((r1 - r0, inp), generator=g, device=device, dtype=torch.float32)
        v = torch.zeros_like(z)
        for _ in range(df):
            e = torch.randn((r1 - r0, inp), generator=g, device=device, dtype=torch.float32)
            v.addcmul_(e, e)
        z.div_(torch.sqrt(v / df)).mul_(scale)
        w[r0:r1] = z.to(dtype)
    return w


def channel_sigma(inp: int, log_std: float, seed: int, device="cpu", hot_frac: float = 0.0,
                  hot_mult: float = 1.0, batch: int | None = None):
    """Per-channel activation std: exp(log_std * N(0,1)) (log_std=0 -> 1), optional hot channels."""
    g = _gen(seed, _SIGMA, device)
    shape = (inp,) if batch is None else (batch, inp)
    if log_std > 0:
        sig = torch.exp(torch.randn(shape, generator=g, device=device) * log_std)
    else:
        sig = torch.ones(shape, device=device)
    n_hot = int(round(hot_frac * inp))
    if n_hot > 0:
        idx = torch.randperm(inp, generator=g, device=device)[:n_hot]
        sig[..., idx] *= hot_mult
    return sig


def activations(tokens: int, sigma: torch.Tensor, seed: int, chunk_index: int = 0,
                device="cpu", dtype=torch.bfloat16):
    """One chunk of calibration activations x_tj = N(0,1) * sigma_j, drawn per (seed, chunk)."""
    g = _gen(seed * 1000 + chunk_index, _X, device)
    x = torch.randn((tokens, sigma.shape[-1]), generator=g, device=device, dtype=torch.float32)
    x.mul_(sigma.to(device))
    return x.to(dtype)


def zipf_counts(n_experts: int, total: int, seed: int, s: float = 1.0) -> np.ndarray:
    """Token counts per expert, proportional to 1/rank^s over a seeded permutation."""
    rng = np.random.Generator(np.random.PCG64(seed * 64 + _ZIPF))
    ranks = rng.permutation(n_experts) + 1
    weights = 1.0 / ranks.astype(np.float64) ** s
    ideal = weights / weights.sum() * (total - n_experts)
    base = np.floor(ideal).astype(np.int64)
    rem = total - n_experts - int(base.sum())
    order = np.argsort(-(ideal - base), kind="stable")
    base[order[:rem]] += 1
    counts = base + 1
    assert int(counts.sum()) == total and counts.min() >= 1
    return counts


@dataclass
class Mode:
    objective: str            # "mse" or "wmse"
    lo: int = 0
    hi: int = 0
    exhaustive: bool = False
    proposal: bool = False    # window around per-group proposal codes, plus the incoming code

    @property
    def label(self) -> str:
        if self.exhaustive:
            return f"{self.objective.upper()} exhaustive(126)"
        if self.proposal:
            return f"{self.objective.upper()} proposal [{self.lo},{self.hi}] + incoming"
        return f"{self.objective.upper()} [{self.lo},{self.hi}]"


@dataclass
class Config:
    name: str
    seed: int
    batch: int
    out: int
    inp: int
    tokens: int
    w_dtype: torch.dtype
    gs_rule: str              # "amax448" | "amax256"
    modes: list = field(default_factory=list)
    chunk_tokens: int = 0     # 0 = one chunk
    description: str = ""

    @property
    def n_weights(self) -> int:
        return self.batch * self.out * self.inp


CONFIGS = {
    "tiny": Config("tiny", 1000, 1, 256, 256, 512, torch.float32, "amax448",
                   [Mode("wmse", -9, 6), Mode("wmse", exhaustive=True), Mode("mse", -3, 7)],
                   description="Tiny layer: W 256x256 fp32, X 512x256 bf16"),
    "attn8b": Config("attn8b", 1001, 1, 4096, 4096, 8192, torch.bfloat16, "amax256",
                     [Mode("mse", -3, 7), Mode("wmse", -8, 7)],
                     description="8B-shaped attention projection: W 4096x4096 bf16, X 8192x4096"),
    "down8b": Config("down8b", 1002, 1, 4096, 14336, 16384, torch.bfloat16, "amax256",
                     [Mode("wmse", -9, 6)],
                     description="8B-shaped MLP down projection: W 4096x14336, X 16384x14336"),
    "moe": Config("moe", 1003, 128, 768, 2048, 262144, torch.bfloat16, "amax448",
                  [Mode("wmse", -9, 6)],
                  description="MoE expert batch: 128 x W 768x2048, X 262144x2048 Zipf-routed"),
    "mlp70b_up": Config("mlp70b_up", 1004, 1, 28672, 8192, 65536, torch.bfloat16, "amax448",
                        [Mode("wmse", -9, 6), Mode("wmse", exhaustive=True)], chunk_tokens=8192,
                        description="70B-shaped MLP up/gate: W 28672x8192, X 65536x8192"),
    "mlp70b_down": Config("mlp70b_down", 1005, 1, 8192, 28672, 65536, torch.bfloat16, "amax448",
                          [Mode("wmse", -9, 6), Mode("wmse", exhaustive=True)], chunk_tokens=8192,
                          description="70B-shaped MLP down: W 8192x28672, X 65536x28672"),
    # The proposal-centred variant of Replay the Curvature (App. D.2: half-window 4 plus the
    # incoming scale) on the 70B up-projection shape. The proposal codes are the max-abs base
    # codes moved by seeded offsets in [-3, 3] (proposal_offsets); the incoming codes are the
    # base codes (the status-quo scale before refinement).
    "mlp70b_up_proposal": Config("mlp70b_up_proposal", 1004, 1, 28672, 8192, 65536,
                                 torch.bfloat16, "amax448", [Mode("wmse", -4, 4, proposal=True)],
                                 chunk_tokens=8192,
                                 description="70B-shaped MLP up/gate, proposal-centred window "
                                             "[-4,4] + incoming scale: W 28672x8192, X 65536x8192"),
}


# Workloads of several matrices measured as one step: the 70B-shaped MLP pair, the up/gate
# projection (28672x8192, X 65536x8192) and the down projection (8192x28672, X 65536x28672),
# each streamed in 8192-token chunks and searched in both of its modes.
GROUPS = {"mlp70b": ("mlp70b_up", "mlp70b_down")}


def workload_configs(name: str) -> list:
    """The configs a named workload covers: one, or every matrix of a group."""
    return [CONFIGS[n] for n in GROUPS.get(name, (name,))]


def proposal_offsets(cfg: Config, shape, device="cpu"):
    """Seeded integer offsets in [-3, 3] that move a group's base code to a synthetic proposal
    (the pages' proposals come from a GPTQ-state quadratic fit that needs trained weights)."""
    g = _gen(cfg.seed, _PROP, device)
    return torch.randint(-3, 4, tuple(shape), generator=g, device=device, dtype=torch.int32)


def make_weights(cfg: Config, device="cpu"):
    """W for a config: [out, in] (or [batch, out, in] for the expert batch)."""
    if cfg.name == "tiny":
        return normal_weights(cfg.out, cfg.inp, 0.02, 0.005, 20.0, cfg.seed, device, torch.float32)
    if cfg.name == "attn8b":
        return normal_weights(cfg.out, cfg.inp, 0.02, 0.001, 30.0, cfg.seed, device)
    if cfg.name == "down8b":
        return student_t_weights(cfg.out, cfg.inp, 4, 0.015, cfg.seed, device)
    if cfg.name == "moe":
        return normal_weights(cfg.out, cfg.inp, 0.02, 0.0, 1.0, cfg.seed, device, batch=cfg.batch)
    if cfg.name.startswith("mlp70b"):
        return student_t_weights(cfg.out, cfg.inp, 5, 0.015, cfg.seed, device)
    raise KeyError(cfg.name)


def make_sigma(cfg: Config, device="cpu"):
    if cfg.name == "tiny":
        return channel_sigma(cfg.inp, 1.0, cfg.seed, device)
    if cfg.name == "attn8b":
        return channel_sigma(cfg.inp, 1.5, cfg.seed, device)
    if cfg.name == "down8b":
        return channel_sigma(cfg.inp, 0.0, cfg.seed, device, hot_frac=0.01, hot_mult=50.0)
    if cfg.name == "moe":
        return channel_sigma(cfg.inp, 1.0, cfg.seed, device, batch=cfg.batch)
    if cfg.name.startswith("mlp70b"):
        return channel_sigma(cfg.inp, 1.5, cfg.seed, device)
    raise KeyError(cfg.name)


def n_chunks(cfg: Config) -> int:
    return 1 if not cfg.chunk_tokens else math.ceil(cfg.tokens / cfg.chunk_tokens)


def make_activation_chunk(cfg: Config, sigma: torch.Tensor, chunk: int, device="cpu"):
    """Chunk `chunk` of X ([chunk_tokens, in]); for the expert batch, the whole routed X
    ([tokens, in], rows grouped by expert) with its segment offsets."""
    if cfg.name == "moe":
        counts = zipf_counts(cfg.batch, cfg.tokens, cfg.seed)
        offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
        X = torch.empty((cfg.tokens, cfg.inp), device=device, dtype=torch.bfloat16)
        for e in range(cfg.batch):
            X[offsets[e]:offsets[e + 1]] = activations(int(counts[e]), sigma[e], cfg.seed, e, device)
        return X, offsets
    T = cfg.chunk_tokens or cfg.tokens
    t0 = chunk * T
    return activations(min(T, cfg.tokens - t0), sigma, cfg.seed, chunk, device), None
