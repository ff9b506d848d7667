"""Checks that pin the AdamW oracle to facts other than itself.

Each ``pin_*`` takes the module (``oracle.adamw`` or a planted-mistake copy of
it) and raises AssertionError when it disagrees with:
- torch.optim.AdamW on the CPU in float64, one optimizer per adapter (each
  adapter has its own hyperparameters and starts at its own step);
- the closed form of the first step from zero state with no decay: the step
  is lr g / (|g| + eps) (the bias-corrected moments are g and g^2);
- a constant gradient: the bias-corrected moments stay g and g^2 at every
  step, so each step moves p by the same amount;
- the unrolled moment recursions m_t = (1-b1) sum_k b1^(t-k) g_k and
  v_t = (1-b2) sum_k b2^(t-k) g_k^2;
- a zero gradient from zero state: only the decoupled decay acts;
- betas of zero: the moments are the current g and g^2 and need no correction;
- step numbers of 0 or less leave everything unchanged;
- per-adapter clipping against torch.nn.utils.clip_grad_norm_ followed by
  torch.optim.AdamW (one adapter clipped, one under its limit, one off), and
  the closed form of a clipped first step.
"""
from __future__ import annotations

import numpy as np


def _rng_case(seed, shapes):
    rng = np.random.default_rng(seed)
    p = [rng.standard_normal(s) * 0.05 for s in shapes]
    g = [rng.standard_normal(s) * 10.0 ** rng.uniform(-4, -1) for s in shapes]
    return rng, p, g


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    den = max(float(np.max(np.abs(b))), 1e-300)
    err = float(np.max(np.abs(a - b))) / den
    assert err <= tol, f"{what}: err {err:.3e} > {tol:.1e}"


def pin_torch_adamw(oa):
    import torch

    hps = [
        dict(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
        dict(lr=4e-5, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.0),
        dict(lr=3e-3, beta1=0.5, beta2=0.9, eps=1e-3, weight_decay=0.3),
    ]
    starts = [0, 2, 1]      # adapter i joins at global step starts[i]
    shapes = [[(8, 4), (4, 16)], [(8, 2), (2, 16)], [(8, 8), (8, 16)]]
    rng = np.random.default_rng(7)
    params = [[rng.standard_normal(s) * 0.05 for s in sh] for sh in shapes]
    m = [[np.zeros(s) for s in sh] for sh in shapes]
    v = [[np.zeros(s) for s in sh] for sh in shapes]
    tparams = [[torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in pi] for pi in params]
    opts = [torch.optim.AdamW(tp, lr=h["lr"], betas=(h["beta1"], h["beta2"]), eps=h["eps"],
                              weight_decay=h["weight_decay"], foreach=False)
            for tp, h in zip(tparams, hps)]
    for gstep in range(5):
        grads = [[rng.standard_normal(s) * 10.0 ** rng.uniform(-3, 0) for s in sh] for sh in shapes]
        hp = []
        for i, h in enumerate(hps):
            t = gstep - starts[i] + 1
            hp.append(dict(h, step=t))
            if t >= 1:
                for tp, g in zip(tparams[i], grads[i]):
                    tp.grad = torch.tensor(g, dtype=torch.float64)
                opts[i].step()
        params, m, v = oa.adamw_step(params, grads, m, v, hp)
        for i in range(len(hps)):
            for k in range(2):
                _close(params[i][k], tparams[i][k].detach().numpy(), 1e-12, f"step {gstep} adapter {i} tensor {k}")
    for i, opt in enumerate(opts):
        for k, tp in enumerate(tparams[i]):
            st = opt.state[tp]
            _close(m[i][k], st["exp_avg"].numpy(), 1e-12, f"m adapter {i} tensor {k}")
            _close(v[i][k], st["exp_avg_sq"].numpy(), 1e-12, f"v adapter {i} tensor {k}")


def pin_first_step_closed_form(oa):
    _, p, g = _rng_case(11, [(16, 8)])
    lr, eps = 2e-4, 1e-8
    z = np.zeros_like(p[0])
    pn, mn, vn = oa.adamw_tensor(p[0], g[0], z, z, lr, 0.9, 0.999, eps, 0.0, 1)
    _close(pn - p[0], -lr * g[0] / (np.abs(g[0]) + eps), 1e-12, "first step")
    _close(mn, 0.1 * g[0], 1e-12, "first m")
    _close(vn, 0.001 * g[0] ** 2, 1e-9, "first v")


def pin_constant_gradient(oa):
    _, p, g = _rng_case(12, [(8, 8)])
    lr, eps = 1e-3, 1e-6
    pc, mc, vc = p[0], np.zeros_like(p[0]), np.zeros_like(p[0])
    per_step = -lr * g[0] / (np.abs(g[0]) + eps)
    for t in range(1, 7):
        pn, mc, vc = oa.adamw_tensor(pc, g[0], mc, vc, lr, 0.9, 0.99, eps, 0.0, t)
        _close(pn - pc, per_step, 1e-9, f"constant gradient, step {t}")
        pc = pn


def pin_unrolled_moments(oa):
    rng, p, _ = _rng_case(13, [(4, 6)])
    b1, b2 = 0.7, 0.9
    gs = [rng.standard_normal((4, 6)) for _ in range(4)]
    pc, mc, vc = p[0], np.zeros((4, 6)), np.zeros((4, 6))
    for t, g in enumerate(gs, start=1):
        pc, mc, vc = oa.adamw_tensor(pc, g, mc, vc, 1e-3, b1, b2, 1e-8, 0.05, t)
    T = len(gs)
    m_ref = (1 - b1) * sum(b1 ** (T - k) * gs[k - 1] for k in range(1, T + 1))
    v_ref = (1 - b2) * sum(b2 ** (T - k) * gs[k - 1] ** 2 for k in range(1, T + 1))
    _close(mc, m_ref, 1e-12, "unrolled m")
    _close(vc, v_ref, 1e-12, "unrolled v")


def pin_zero_grad_pure_decay(oa):
    _, p, _ = _rng_case(14, [(8, 4)])
    z = np.zeros_like(p[0])
    lr, wd = 5e-3, 0.2
    pn, mn, vn = oa.adamw_tensor(p[0], z, z, z, lr, 0.9, 0.999, 1e-8, wd, 5)
    _close(pn, p[0] * (1 - lr * wd), 1e-14, "pure decay")
    assert not np.any(mn) and not np.any(vn), "moments of a zero gradient must stay zero"


def pin_zero_betas(oa):
    _, p, g = _rng_case(15, [(8, 4)])
    rng = np.random.default_rng(3)
    m0, v0 = rng.standard_normal((8, 4)), rng.uniform(0, 1, (8, 4))
    lr, eps, wd = 1e-3, 1e-7, 0.1
    for t in (1, 9):
        pn, mn, vn = oa.adamw_tensor(p[0], g[0], m0, v0, lr, 0.0, 0.0, eps, wd, t)
        _close(mn, g[0], 1e-15, "b1 = 0 keeps only g")
        _close(vn, g[0] ** 2, 1e-15, "b2 = 0 keeps only g^2")
        _close(pn, p[0] * (1 - lr * wd) - lr * g[0] / (np.abs(g[0]) + eps), 1e-13, "zero betas")


def pin_skip(oa):
    _, p, g = _rng_case(16, [(8, 4)])
    rng = np.random.default_rng(4)
    m0, v0 = rng.standard_normal((8, 4)), rng.uniform(0, 1, (8, 4))
    for t in (0, -3):
        pn, mn, vn = oa.adamw_tensor(p[0], g[0], m0, v0, 1e-3, 0.9, 0.999, 1e-8, 0.1, t)
        assert np.array_equal(pn, p[0]) and np.array_equal(mn, m0) and np.array_equal(vn, v0), \
            f"step {t} must leave the adapter unchanged"


def pin_elements_match_whole(oa):
    _, p, g = _rng_case(17, [(16, 12)])
    rng = np.random.default_rng(5)
    m0, v0 = rng.standard_normal((16, 12)) * 1e-3, rng.uniform(0, 1e-6, (16, 12))
    whole = oa.adamw_tensor(p[0], g[0], m0, v0, 1e-3, 0.9, 0.999, 1e-8, 0.1, 3)
    idx = rng.choice(16 * 12, 40, replace=False)
    part = oa.adamw_elements(p[0], g[0], m0, v0, 1e-3, 0.9, 0.999, 1e-8, 0.1, 3, idx)
    for a, b, name in zip(part, whole, "pmv"):
        assert np.array_equal(a, b.reshape(-1)[idx]), f"sampled {name} differs from the whole update"


def pin_clipping_vs_torch(oa):
    import torch
    hps = [dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, max_grad_norm=0.05),
           dict(lr=2e-4, beta1=0.8, beta2=0.95, eps=1e-6, weight_decay=0.0, max_grad_norm=1e3),
           dict(lr=5e-4, beta1=0.9, beta2=0.99, eps=1e-8, weight_decay=0.1, max_grad_norm=0.0)]
    shapes = [[(8, 4), (4, 16)], [(8, 2), (2, 16)], [(8, 8), (8, 16)]]
    rng = np.random.default_rng(21)
    params = [[rng.standard_normal(sh) * 0.05 for sh in s] for s in shapes]
    m = [[np.zeros(sh) for sh in s] for s in shapes]
    v = [[np.zeros(sh) for sh in s] for s in shapes]
    tps = [[torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in pi] for pi in params]
    opts = [torch.optim.AdamW(tp, lr=h["lr"], betas=(h["beta1"], h["beta2"]), eps=h["eps"],
                              weight_decay=h["weight_decay"], foreach=False) for tp, h in zip(tps, hps)]
    for t in range(1, 4):
        grads = [[rng.standard_normal(sh) * 0.1 for sh in s] for s in shapes]
        for i, h in enumerate(hps):
            for tp, g in zip(tps[i], grads[i]):
                tp.grad = torch.tensor(g, dtype=torch.float64)
            if h["max_grad_norm"] > 0:
                torch.nn.utils.clip_grad_norm_(tps[i], h["max_grad_norm"])
            opts[i].step()
        params, m, v = oa.adamw_step(params, grads, m, v, [dict(h, step=t) for h in hps])
        for i in range(3):
            for k in range(2):
                _close(params[i][k], tps[i][k].detach().numpy(), 1e-12, f"clipped step {t} adapter {i} tensor {k}")


def pin_clipped_first_step_moments(oa):
    rng = np.random.default_rng(22)
    g = [rng.standard_normal((6, 3)), rng.standard_normal((3, 5))]
    norm = np.sqrt(sum(np.sum(x ** 2) for x in g))
    mx = 0.25 * norm
    z = [np.zeros_like(x) for x in g]
    _, m1, v1 = oa.adamw_step([[np.ones_like(x) for x in g]], [g], [z], [z],
                              [dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0, step=1,
                                    max_grad_norm=mx)])
    c = mx / (norm + 1e-6)
    for k in range(2):
        _close(m1[0][k], 0.1 * c * g[k], 1e-12, "clipped first moment")
        _close(v1[0][k], 0.001 * (c * g[k]) ** 2, 1e-10, "clipped second moment")


ALL_PINS = [pin_clipping_vs_torch, pin_clipped_first_step_moments, pin_torch_adamw, pin_first_step_closed_form, pin_constant_gradient, pin_unrolled_moments,
            pin_zero_grad_pure_decay, pin_zero_betas, pin_skip, pin_elements_match_whole]
