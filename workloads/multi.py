"""Seeded inputs of layers whose projections share one input (q/k/v, gate/up).

The projections of a fused group read the same X.  Every other tensor of
projection q is drawn exactly as for the unfused projection (same generators,
same distributions), then laid out concatenated along the output: W0 is
[d_in][sum of widths], dY is [T][sum of widths], and adapter i keeps its own
A_iq, B_iq and scale s_iq = 16 / r_iq per projection.  X is the group's first
projection's X.  No arithmetic of the layer lives here.
"""
from __future__ import annotations

import numpy as np

from .configs import Workload, STD_X, STD_DY, STD_W0, STD_B, std_a
from .tensors import _draw, _rng, _TENSOR_IDS

# How the seven projections of a decoder layer group by shared input.
LAYER_GROUPS = {
    "llama3_8b_layer": [("qkv", [0, 1, 2]), ("o", [3]), ("gate_up", [4, 5]), ("down", [6])],
}


def host_multi(seed, d_in, widths, ranks, tokens, dtype="bf16", scales=None):
    """Host arrays for a small fused layer: X [T][d_in], W0 [d_in][D],
    dY [T][D], A[i][q] [d_in][r_iq], B[i][q] [r_iq][d_q], scales[i][q],
    offsets [n+1].  bf16 tensors are uint16 bit patterns."""
    n, P = len(tokens), len(widths)
    off = np.zeros(n + 1, dtype=np.int64)
    off[1:] = np.cumsum(np.asarray(tokens, dtype=np.int64))
    T = int(off[-1])
    X = _draw(_rng(seed, 0, "X"), (T, d_in), STD_X, dtype)
    W0 = np.concatenate([_draw(_rng(seed, q, "W0"), (d_in, widths[q]), STD_W0, dtype) for q in range(P)], axis=1)
    dY = np.concatenate([_draw(_rng(seed, q, "dY"), (T, widths[q]), STD_DY, dtype) for q in range(P)], axis=1)
    A = [[_draw(_rng(seed, q, "A", i), (d_in, ranks[i][q]), std_a(d_in), dtype) for q in range(P)]
         for i in range(n)]
    B = [[_draw(_rng(seed, q, "B", i), (ranks[i][q], widths[q]), STD_B, dtype) for q in range(P)]
         for i in range(n)]
    if scales is None:
        scales = [[16.0 / ranks[i][q] for q in range(P)] for i in range(n)]
    return dict(X=np.ascontiguousarray(X), W0=np.ascontiguousarray(W0), dY=np.ascontiguousarray(dY), A=A,
                B=B, scales=scales, offsets=off, widths=list(widths), ranks=[list(r) for r in ranks],
                d_in=d_in, dtype=dtype)


def device_multi(w: Workload, projs, seed=None, device="cuda", sets=1):
    """A fused group of a bf16 workload drawn on the device: the projections
    ``projs`` (indices into w.projections, same d_in) sharing the first
    one's X; the same adapters (ranks, tokens) on every projection.  Returns
    torch tensors W0 [d_in][D], X and dY lists of ``sets``, A and B nested
    [adapter][projection], and host lists of scales, ranks, widths."""
    import torch

    s = w.seed if seed is None else seed
    d_in = w.projections[projs[0]].d_in
    assert all(w.projections[q].d_in == d_in for q in projs) and w.dtype == "bf16"
    T = w.T

    def draw(proj, shape, std, tid, idx=0):
        g = torch.Generator(device=device)
        g.manual_seed((s * 1000003 + proj * 7919 + _TENSOR_IDS[tid] * 104729 + idx * 31) & 0x7FFFFFFF)
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        t.mul_(std)
        return t.to(torch.bfloat16)

    widths = [w.projections[q].d_out for q in projs]
    W0 = torch.cat([draw(q, (d_in, w.projections[q].d_out), STD_W0, "W0") for q in projs], dim=1).contiguous()
    X = [draw(projs[0], (T, d_in), STD_X, "X", k) for k in range(sets)]
    dY = [torch.cat([draw(q, (T, w.projections[q].d_out), STD_DY, "dY", k) for q in projs], dim=1).contiguous()
          for k in range(sets)]
    A = [[draw(q, (d_in, r), std_a(d_in), "A", i) for q in projs] for i, r in enumerate(w.ranks)]
    B = [[draw(q, (r, w.projections[q].d_out), STD_B, "B", i) for q in projs] for i, r in enumerate(w.ranks)]
    P = len(projs)
    return {
        "W0": W0, "X": X, "dY": dY, "A": A, "B": B,
        "scales": [[w.scales[i]] * P for i in range(w.n)],
        "ranks": [[r] * P for r in w.ranks],
        "widths": widths, "offsets": w.seg_offsets(), "d_in": d_in,
    }
