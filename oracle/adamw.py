"""Per-adapter AdamW update in float64 -- TEST INFRASTRUCTURE ONLY.

Parity pinned: see tests/pins_adamw.py (torch.optim.AdamW in float64 with
one parameter group per adapter, the closed form of the first step, the
closed form of a constant gradient, pure decay under a zero gradient, the
degenerate betas, and the skip rule).

What it follows (PLoRA: Efficient Concurrent LoRA Training for Large Language
Models):
- §2.4: every packed adapter keeps its own parameters and its own optimizer
  state, so the update of one adapter never reads another's.
- §8 (LoRA memory constraints): the optimizer is AdamW, whose state per
  trained parameter is a first moment (momentum) and a second moment
  (velocity) beside the gradient.
- §2.2 and §11.1 (Table 4): the learning rate is a per-configuration knob, so
  every adapter brings its own hyperparameters and its own step count.

The pages do not write AdamW out.  The update used is Adam (Kingma and Ba,
Algorithm 1) with the weight decay decoupled from the gradient (Loshchilov
and Hutter, Algorithm 2), the decay multiplied by the learning rate as
torch.optim.AdamW applies it (PLoRA runs inside torchtune, a PyTorch
library).  For one adapter with learning rate lr, betas b1 and b2, epsilon
eps, weight decay wd and step number t >= 1, every trained element p with
gradient g and state (m, v) becomes:

    p <- p (1 - lr wd)
    m <- b1 m + (1 - b1) g
    v <- b2 v + (1 - b2) g^2
    p <- p - lr (m / (1 - b1^t)) / (sqrt(v / (1 - b2^t)) + eps)

An adapter whose step number is 0 or less is not updated: its parameters and
state are returned unchanged.  Inputs are upcast to float64 and nothing is
rounded in between.

Optional per-adapter gradient clipping (max_grad_norm > 0): before the update,
every gradient of the adapter is multiplied by min(1, max_grad_norm /
(||g|| + 1e-6)), ||g|| the 2-norm over all of the adapter's trained tensors
together -- the rule of torch.nn.utils.clip_grad_norm_, applied to each
adapter (each job) on its own.
"""
from __future__ import annotations

import numpy as np


def adamw_tensor(p, g, m, v, lr, beta1, beta2, eps, weight_decay, step):
    """One AdamW update of one tensor; returns (p, m, v) as new float64 arrays."""
    p = np.asarray(p, dtype=np.float64).copy()
    g = np.asarray(g, dtype=np.float64)
    m = np.asarray(m, dtype=np.float64).copy()
    v = np.asarray(v, dtype=np.float64).copy()
    t = int(step)
    if t <= 0:
        return p, m, v
    lr, beta1, beta2 = float(lr), float(beta1), float(beta2)
    eps, weight_decay = float(eps), float(weight_decay)
    p = p * (1.0 - lr * weight_decay)
    m = beta1 * m + (1.0 - beta1) * g
    v = beta2 * v + (1.0 - beta2) * g * g
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    p = p - lr * m_hat / (np.sqrt(v_hat) + eps)
    return p, m, v


def clip_coef(grads, max_grad_norm):
    """The factor one adapter's gradients are multiplied by (1 when clipping
    is off, max_grad_norm <= 0)."""
    mx = float(max_grad_norm)
    if mx <= 0.0:
        return 1.0
    norm = np.sqrt(sum(float(np.sum(np.asarray(g, dtype=np.float64) ** 2)) for g in grads))
    return min(1.0, mx / (norm + 1e-6))


def adamw_step(params, grads, m, v, hparams):
    """One AdamW step of every adapter.

    params, grads, m, v: per adapter, a list of the adapter's trained tensors
    (for the LoRA layer: [A_i, B_i]).  hparams: per adapter, a mapping with
    lr, beta1, beta2, eps, weight_decay, step and optionally max_grad_norm
    (clipping over the adapter's tensors together).  Returns new lists
    (params, m, v) of float64 arrays, nested as the inputs.
    """
    out_p, out_m, out_v = [], [], []
    for i, h in enumerate(hparams):
        pi, mi, vi = [], [], []
        c_i = clip_coef(grads[i], h.get("max_grad_norm", 0.0)) if int(h["step"]) > 0 else 1.0
        for p, g, mm, vv in zip(params[i], grads[i], m[i], v[i]):
            a, b, c = adamw_tensor(p, np.asarray(g, dtype=np.float64) * c_i, mm, vv, h["lr"], h["beta1"],
                                   h["beta2"], h["eps"], h["weight_decay"], h["step"])
            pi.append(a)
            mi.append(b)
            vi.append(c)
        out_p.append(pi)
        out_m.append(mi)
        out_v.append(vi)
    return out_p, out_m, out_v


def adamw_elements(p, g, m, v, lr, beta1, beta2, eps, weight_decay, step, idx):
    """The update at flat element indices ``idx`` only (for sampled checks of
    tensors too large to update whole in float64)."""
    idx = np.asarray(idx)
    take = lambda a: np.asarray(a).reshape(-1)[idx]
    return adamw_tensor(take(p), take(g), take(m), take(v), lr, beta1, beta2, eps,
                        weight_decay, step)
