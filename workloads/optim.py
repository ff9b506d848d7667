"""Seeded inputs of the per-adapter optimizer step.

Master weights, per-step gradients and per-adapter hyperparameters, drawn in
fp32 from ``default_rng(SeedSequence(...))``; the same values go to the
device and to the oracle.  No arithmetic of the update lives here.

Distributions: A_i ~ N(0, 1/d_in) and B_i ~ N(0, 0.01) as in the layer's
workloads; gradients ~ N(0, 1) times a per-tensor magnitude 10^U(-4, -1).
Learning rates are log-uniform in [4e-5, 1e-3] (the PLoRA page's best
configurations in Table 4 use 4e-5 and 1e-4); betas, eps and weight decay
are drawn from common settings, including the degenerate beta of 0.
"""
from __future__ import annotations

import numpy as np

from .configs import STD_B, std_a

BETA1 = (0.9, 0.9, 0.8, 0.0)
BETA2 = (0.999, 0.999, 0.95, 0.0)
EPS = (1e-8, 1e-6)
WEIGHT_DECAY = (0.0, 0.01, 0.1)


def _rng(seed, *ids):
    return np.random.default_rng(np.random.SeedSequence([seed, 77, *ids]))


def masters(ranks, d_in, d_out, seed):
    """fp32 A_i [d_in][r_i] and B_i [r_i][d_out] per adapter."""
    A, B = [], []
    for i, r in enumerate(int(v) for v in ranks):
        A.append(_rng(seed, 1, i).standard_normal((d_in, r), dtype=np.float32) * np.float32(std_a(d_in)))
        B.append(_rng(seed, 2, i).standard_normal((r, d_out), dtype=np.float32) * np.float32(STD_B))
    return A, B


def gradients(ranks, d_in, d_out, seed, step):
    """fp32 gradients of step ``step`` (0-based) for every A_i and B_i."""
    dA, dB = [], []
    for i, r in enumerate(int(v) for v in ranks):
        for shape, out, k in (((d_in, r), dA, 3), ((r, d_out), dB, 4)):
            g = _rng(seed, k, i, step)
            mag = np.float32(10.0 ** g.uniform(-4.0, -1.0))
            out.append(g.standard_normal(shape, dtype=np.float32) * mag)
    return dA, dB


def hyperparameters(n, seed):
    """Per adapter: lr, beta1, beta2, eps, weight_decay (as fp32 values) and
    the global step at which the adapter starts (0 for most; some later, so
    their step numbers stay <= 0 and they are skipped for a while)."""
    g = _rng(seed, 5)
    out = []
    for i in range(n):
        out.append(dict(
            lr=float(np.float32(10.0 ** g.uniform(np.log10(4e-5), -3.0))),
            beta1=float(np.float32(BETA1[g.integers(len(BETA1))])),
            beta2=float(np.float32(BETA2[g.integers(len(BETA2))])),
            eps=float(np.float32(EPS[g.integers(len(EPS))])),
            weight_decay=float(np.float32(WEIGHT_DECAY[g.integers(len(WEIGHT_DECAY))])),
            start=int(g.choice([0, 0, 0, 1, 2])),
        ))
    return out


def step_hparams(hps, global_step):
    """The hyperparameters of global step ``global_step`` (0-based): each
    adapter's own step number is global_step - start + 1."""
    return [dict({k: v for k, v in h.items() if k != "start"}, step=global_step - h["start"] + 1)
            for h in hps]
