"""Seeded synthetic held-out data for Sequential Temperature Scaling.

Random numbers only.  An instance n has, per draft position k, a latent logit
eta_{n,k} ~ N(mu, s) of the true conditional survival probability; the
confidence head reports t_{n,k} = kappa_k * eta_{n,k} + N(0, noise) (kappa_k > 1:
an overconfident head, as the pages report for the raw head); the label
y_{n,k} = 1 while every position 1 .. k has survived, each with probability
sigmoid(eta_{n,k}).  No trained head or validation set exists here, so this
stands in for one.
"""

from __future__ import annotations

import numpy as np
import torch


def make_sts_inputs(N: int, G: int, seed: int = 0, kappa=None, mu: float = 1.5, s: float = 1.5,
                    noise: float = 0.3, device="cpu"):
    rng = np.random.default_rng(int(seed) + 9100)
    if kappa is None:
        kappa = 1.6 + 1.4 * rng.random(G)           # per-position overconfidence in [1.6, 3.0)
    kappa = np.asarray(kappa, dtype=np.float64)
    eta = rng.normal(mu, s, (N, G))
    t = (kappa[None, :] * eta + rng.normal(0.0, noise, (N, G))).astype(np.float32)
    survive = rng.random((N, G)) < 1.0 / (1.0 + np.exp(-eta))
    y = np.cumprod(survive, axis=1).astype(np.uint8)
    return torch.from_numpy(t).to(device), torch.from_numpy(y).to(device), kappa


def tau_grid(n: int = 256, lo: float = 0.25, hi: float = 8.0, device="cpu") -> torch.Tensor:
    """Geometric grid of n temperatures from lo to hi (float64)."""
    return torch.from_numpy(np.exp(np.linspace(np.log(lo), np.log(hi), n))).to(device)
