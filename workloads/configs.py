"""Seeded generators for the five verification workloads.

Every tensor is produced by torch's seeded generator on the requested device
(CPU for oracle-only checks, the GPU for anything the HIP path consumes).  The
recipes, all sizes and the readings behind them are listed in the repository's
design notes; the short form:

  tiny       B=1,    gamma=4,  V=1000,   fp32  target N(0,2); draft = target + N(0,0.5); T=1
  mid        B=32,   gamma=16, V=151936, bf16  target N(0,3) + 8 on one random token per row;
                                                draft_k = target_k + N(0, 0.3 + 0.08 k)  (k from 0)
  scheduled  B=256,  gamma=16, V=151936, bf16  logits as `tiny`: target N(0,2), draft = target + N(0,0.5);
                                                c_k = sigmoid(N(1.5-0.15k, 1)), k from 1;
                                                8-point concave throughput table; budget 2048 tokens
  greedy     B=512,  gamma=16, V=129280, bf16  target N(0,3); T=0; x_k = target argmax w.p. 0.9^k
                                                (k from 1) else uniform over the vocabulary
  mixed      B=1024, gamma=8,  V=129280, bf16  target N(0,3); draft = target + N(0,0.8);
                                                T ~ U[0.6,1.2]; top-k 50; per-request seeds

The second argument of N(.,.) is a standard deviation throughout.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# name -> recipe.  `noise` is the draft noise std per position k (0-based).
CONFIGS = {
    "tiny": dict(B=1, gamma=4, V=1000, dtype="f32", target_std=2.0, spike=0.0,
                 noise=("const", 0.5), temp=("const", 1.0), top_k=0, seeds="zero", seed=1001),
    "mid": dict(B=32, gamma=16, V=151936, dtype="bf16", target_std=3.0, spike=8.0,
                noise=("linear", 0.3, 0.08), temp=("const", 1.0), top_k=0, seeds="zero", seed=1002),
    "scheduled": dict(B=256, gamma=16, V=151936, dtype="bf16", target_std=2.0, spike=0.0,
                      noise=("const", 0.5), temp=("const", 1.0), top_k=0, seeds="zero",
                      seed=1003, budget=2048, table_seed=3003),
    "greedy": dict(B=512, gamma=16, V=129280, dtype="bf16", target_std=3.0, spike=0.0,
                   noise=None, temp=("const", 0.0), top_k=0, seeds="zero", seed=1004,
                   greedy_match=0.9),
    "mixed": dict(B=1024, gamma=8, V=129280, dtype="bf16", target_std=3.0, spike=0.0,
                  noise=("const", 0.8), temp=("uniform", 0.6, 1.2), top_k=50, seeds="random",
                  seed=1005),
}

TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    gamma: int
    V: int
    dtype: str                              # "f32" | "bf16"
    target: torch.Tensor                    # [B, gamma+1, V]
    draft: Optional[torch.Tensor]           # [B, gamma, V]; None for greedy-only inputs
    draft_tokens: torch.Tensor              # [B, gamma] int32
    temperature: torch.Tensor               # [B] float32 (0 = greedy rule)
    top_k: Optional[torch.Tensor]           # [B] int32 or None (off)
    seed: torch.Tensor                      # [B] int64 holding the uint64 bit pattern
    lengths: Optional[torch.Tensor] = None  # [B] int32 or None (= gamma)
    conf: Optional[torch.Tensor] = None     # [B, gamma] float32 in [0,1]
    sps: Optional[np.ndarray] = None        # float64 dense cost table, index = batch tokens
    budget: Optional[int] = None            # verify budget in batch tokens

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _noise_std(noise, k: int) -> float:
    if noise is None:
        return 0.0
    if noise[0] == "const":
        return float(noise[1])
    if noise[0] == "linear":
        return float(noise[1]) + float(noise[2]) * k
    raise ValueError(noise)


def sample_draft_tokens(draft: torch.Tensor, temperature: torch.Tensor,
                        top_k: Optional[torch.Tensor], gen: torch.Generator) -> torch.Tensor:
    """Simulated drafter: x_k ~ softmax(z/T) over the top-k set (ties kept), by Gumbel-max.

    draft: [B, G, V] logits.  Returns int32 [B, G].  Processed one request at a
    time to bound the fp32 transient.
    """
    B, G, V = draft.shape
    out = torch.empty((B, G), dtype=torch.int32, device=draft.device)
    for i in range(B):
        z = draft[i].float()
        T = float(temperature[i])
        if T <= 0.0:
            out[i] = torch.argmax(z, dim=-1).to(torch.int32)
            continue
        if top_k is not None and 0 < int(top_k[i]) < V:
            kth = torch.topk(z, int(top_k[i]), dim=-1).values[:, -1:]
            z = torch.where(z >= kth, z, torch.full_like(z, -math.inf))
        u = torch.rand(z.shape, generator=gen, device=z.device, dtype=torch.float32)
        u = u.clamp_(min=1e-12, max=1.0 - 1e-7)
        gumbel = -torch.log(-torch.log(u))
        out[i] = torch.argmax(z / T + gumbel, dim=-1).to(torch.int32)
    return out


def make_confidences(B: int, gamma: int, seed: int, device="cpu") -> torch.Tensor:
    """c_{i,k} = sigmoid(N(1.5 - 0.15 k, 1)), k = 1..gamma, in float32."""
    g = _gen("cpu", seed)
    k = torch.arange(1, gamma + 1, dtype=torch.float64)
    mean = 1.5 - 0.15 * k
    x = torch.randn((B, gamma), generator=g, dtype=torch.float64) + mean
    return torch.sigmoid(x).to(torch.float32).to(device)


def make_sps_table(table_len: int, seed: int) -> np.ndarray:
    """Dense engine cost table SPS[b] in steps/s for a forward batch of b tokens.

    Eight (batch tokens -> tokens/s) points at x_j = round(256 * 32^(j/7)),
    throughput T_j = Y (1 - exp(-x_j / X0)) with Y ~ U[5e4, 2e5] and
    X0 ~ U[1e3, 4e3] (concave, increasing).  T(b) is piecewise linear between
    the points and held constant beyond the ends; SPS[b] = T(b) / b, SPS[0] = 0.
    """
    rng = np.random.default_rng(seed)
    Y = rng.uniform(5e4, 2e5)
    X0 = rng.uniform(1e3, 4e3)
    xs = np.array([round(256 * 32 ** (j / 7)) for j in range(8)], dtype=np.float64)
    ts = Y * (1.0 - np.exp(-xs / X0))
    b = np.arange(table_len, dtype=np.float64)
    tput = np.interp(b, xs, ts)
    sps = np.zeros(table_len, dtype=np.float64)
    sps[1:] = tput[1:] / b[1:]
    return sps


def _make_logits(B, gamma, V, cfg, device, gen):
    """Target [B, gamma+1, V] and draft [B, gamma, V] (or None) in the config dtype."""
    dt = TORCH_DTYPES[cfg["dtype"]]
    target = torch.empty((B, gamma + 1, V), dtype=dt, device=device)
    draft = None
    if cfg["noise"] is not None:
        draft = torch.empty((B, gamma, V), dtype=dt, device=device)
    chunk = max(1, (1 << 26) // max(1, (gamma + 1) * V))
    for i0 in range(0, B, chunk):
        i1 = min(B, i0 + chunk)
        n = i1 - i0
        t = torch.randn((n, gamma + 1, V), generator=gen, device=device) * cfg["target_std"]
        if cfg["spike"]:
            idx = torch.randint(V, (n, gamma + 1, 1), generator=gen, device=device)
            t.scatter_add_(2, idx, torch.full((n, gamma + 1, 1), float(cfg["spike"]), device=device))
        target[i0:i1] = t.to(dt)
        if draft is not None:
            d = t[:, :gamma].clone()
            for k in range(gamma):
                s = _noise_std(cfg["noise"], k)
                d[:, k] += torch.randn((n, V), generator=gen, device=device) * s
            draft[i0:i1] = d.to(dt)
        del t
    return target, draft


def _temperatures(B, cfg, gen, device):
    kind = cfg["temp"]
    if kind[0] == "const":
        return torch.full((B,), float(kind[1]), dtype=torch.float32, device=device)
    lo, hi = kind[1], kind[2]
    u = torch.rand((B,), generator=gen, device=device, dtype=torch.float64)
    return (lo + (hi - lo) * u).to(torch.float32)


def _seeds(B, cfg, seed, device):
    if cfg["seeds"] == "zero":
        return torch.zeros((B,), dtype=torch.int64, device=device)
    rng = np.random.default_rng(seed + 4000)
    s = rng.integers(0, 2 ** 64, size=B, dtype=np.uint64)
    return torch.from_numpy(s.view(np.int64).copy()).to(device)


def make_greedy_draft_tokens(target: torch.Tensor, match: float, gen: torch.Generator) -> torch.Tensor:
    """x_k = argmax of target row k with probability match^k (k from 1), else uniform."""
    B, G1, V = target.shape
    G = G1 - 1
    am = torch.argmax(target[:, :G].float() if target.dtype != torch.float32 else target[:, :G], dim=-1)
    k = torch.arange(1, G + 1, device=target.device, dtype=torch.float64)
    p = match ** k
    coin = torch.rand((B, G), generator=gen, device=target.device, dtype=torch.float64)
    rnd = torch.randint(V, (B, G), generator=gen, device=target.device)
    return torch.where(coin < p, am, rnd).to(torch.int32)


def make_workload(name: str, device="cpu", B: Optional[int] = None, gamma: Optional[int] = None,
                  V: Optional[int] = None, seed: Optional[int] = None,
                  with_schedule: Optional[bool] = None) -> Workload:
    """Build a named workload, optionally scaled down (same recipe, other sizes)."""
    cfg = dict(CONFIGS[name])
    B = cfg["B"] if B is None else int(B)
    gamma = cfg["gamma"] if gamma is None else int(gamma)
    V = cfg["V"] if V is None else int(V)
    seed = cfg["seed"] if seed is None else int(seed)
    gen = _gen(device, seed)
    target, draft = _make_logits(B, gamma, V, cfg, device, gen)
    temperature = _temperatures(B, cfg, gen, device)
    top_k = None
    if cfg["top_k"]:
        top_k = torch.full((B,), int(cfg["top_k"]), dtype=torch.int32, device=device)
    if name == "greedy":
        tokens = make_greedy_draft_tokens(target, cfg["greedy_match"], gen)
    else:
        tokens = sample_draft_tokens(draft, temperature, top_k, gen)
    w = Workload(name=name, B=B, gamma=gamma, V=V, dtype=cfg["dtype"], target=target, draft=draft,
                 draft_tokens=tokens, temperature=temperature, top_k=top_k,
                 seed=_seeds(B, cfg, seed, device))
    if with_schedule is None:
        with_schedule = "budget" in cfg
    if with_schedule:
        w.conf = make_confidences(B, gamma, seed + 2000, device)
        w.sps = make_sps_table(B * (gamma + 1) + 1, cfg.get("table_seed", seed + 3000))
        budget = cfg.get("budget", 2048)
        # A scaled-down batch keeps the same budget-per-request ratio (2048 / 256 = 8).
        if B != cfg["B"]:
            budget = max(B, int(round(budget * B / cfg["B"])))
        w.budget = budget
    return w


def make_verify_inputs(name: str, device="cpu", **kw) -> Workload:
    return make_workload(name, device, **kw)


def make_greedy_inputs(device="cpu", **kw) -> Workload:
    return make_workload("greedy", device, **kw)
