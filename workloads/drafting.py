"""Seeded synthetic inputs for the Markov-head draft sampler.

Only random numbers: base logits U from the parallel stage, the Markov head's
embedding table W1 and projection W2 (stored token-major, W2t [V, r]), anchor
tokens, temperatures, seeds, hidden states and the confidence head's weight.
No trained weights exist here, so the weights are drawn at the scale that gives
the transition bias a standard deviation of about one logit.

  gaussian  U: N(0, 3) + 8 on one random token per row (the verification
            workloads' logit recipe), bf16 or fp32; W1 ~ N(0, 1); W2t ~
            N(0, 1/sqrt(r)); h ~ N(0, 1); w ~ N(0, 1/sqrt(d + r))
  grid      every value on a coarse binary grid, so that any fp32 evaluation
            of U + W1[x] W2 is exact: W1, W2t in {-4 .. 4} / 16; U = a
            multiple of 1/8 in [-31, 31] (N(0, 3) rounded, + 8 on one token);
            h in {-8 .. 8} / 8; w in {-8 .. 8} / 64

Temperatures: "mixed" draws T ~ U[0.6, 1.2] with every fifth request greedy
(T = 0); a float sets every request to that value.
"""

from __future__ import annotations

import dataclasses
from typing import Optional, Union

import numpy as np
import torch

_DT = {"bf16": torch.bfloat16, "f32": torch.float32}


@dataclasses.dataclass
class DraftInputs:
    B: int
    gamma: int
    V: int
    r: int
    d: int
    dtype: str
    base: torch.Tensor         # [B, gamma, V]
    W1: torch.Tensor           # [V, r] bf16
    W2t: torch.Tensor          # [V, r] bf16
    anchor: torch.Tensor       # [B] int32
    temperature: torch.Tensor  # [B] float32
    seed: torch.Tensor         # [B] int64 (uint64 bit patterns)
    hidden: Optional[torch.Tensor]   # [B, gamma, d] (dtype) or None
    conf_w: Optional[torch.Tensor]   # [d + r] float32 or None


def make_draft_inputs(B: int, gamma: int, V: int, r: int = 256, d: int = 0, dtype: str = "bf16",
                      kind: str = "gaussian", temperature: Union[str, float] = "mixed", seed: int = 0,
                      device="cpu", conf: bool = True) -> DraftInputs:
    dt = _DT[dtype]
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) + 7000)
    base = torch.empty((B, gamma, V), dtype=dt, device=device)
    chunk = max(1, (1 << 26) // max(1, gamma * V))
    for i0 in range(0, B, chunk):
        n = min(B, i0 + chunk) - i0
        u = torch.randn((n, gamma, V), generator=g, device=device) * 3.0
        idx = torch.randint(V, (n, gamma, 1), generator=g, device=device)
        u.scatter_add_(2, idx, torch.full((n, gamma, 1), 8.0, device=device))
        if kind == "grid":
            u = torch.clamp(torch.round(u * 8.0) / 8.0, -31.0, 31.0)
        base[i0:i0 + n] = u.to(dt)
    if kind == "grid":
        W1 = (torch.randint(-4, 5, (V, r), generator=g, device=device).float() / 16.0).to(torch.bfloat16)
        W2t = (torch.randint(-4, 5, (V, r), generator=g, device=device).float() / 16.0).to(torch.bfloat16)
    else:
        W1 = torch.randn((V, r), generator=g, device=device).to(torch.bfloat16)
        W2t = (torch.randn((V, r), generator=g, device=device) / float(np.sqrt(r))).to(torch.bfloat16)
    anchor = torch.randint(V, (B,), generator=g, device=device).to(torch.int32)
    if temperature == "mixed":
        T = 0.6 + 0.6 * torch.rand((B,), generator=g, device=device, dtype=torch.float64)
        T[::5] = 0.0
        T = T.to(torch.float32)
    else:
        T = torch.full((B,), float(temperature), dtype=torch.float32, device=device)
    rng = np.random.default_rng(int(seed) + 7001)
    s = torch.from_numpy(rng.integers(0, 2 ** 64, size=B, dtype=np.uint64).view(np.int64).copy()).to(device)
    hidden = conf_w = None
    if conf:
        if kind == "grid":
            if d:
                hidden = (torch.randint(-8, 9, (B, gamma, d), generator=g, device=device).float() / 8.0).to(dt)
            conf_w = torch.randint(-8, 9, (d + r,), generator=g, device=device).float() / 64.0
        else:
            if d:
                hidden = torch.randn((B, gamma, d), generator=g, device=device).to(dt)
            conf_w = torch.randn((d + r,), generator=g, device=device) / float(np.sqrt(d + r))
    return DraftInputs(B=B, gamma=gamma, V=V, r=r, d=d, dtype=dtype, base=base, W1=W1, W2t=W2t, anchor=anchor,
                       temperature=T, seed=s, hidden=hidden, conf_w=conf_w)
