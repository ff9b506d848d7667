"""Packed multi-LoRA over several projections that share one input, in
float64 -- TEST INFRASTRUCTURE ONLY.

Parity pinned: see tests/pins_multi.py (one projection reduces to the
single-projection oracle; each projection equals an independent packed layer
and dX is their sum; torch float64 autograd of the block-diagonal form; pure
Python loops on tiny shapes).

What it follows (PLoRA: Efficient Concurrent LoRA Training for Large Language
Models):
- §8 (LoRA memory constraints): an adapter can target the Q, K, V and output
  projections of an attention block and the up, gate and down projections of
  an MLP block.  Q, K and V read the same input, and so do gate and up.
- §9.2: adapters are concatenated, and the token axis is sequence length
  times batch size.
- §2.1 and §2.4: for every (adapter, projection) pair the computation is
  exactly standard LoRA with that pair's own A, B and scale.

Projection p owns output columns [c_p, c_{p+1}) of the concatenated output
(widths d_p, D = sum d_p) and of the concatenated frozen weight
W0 = [W0_1 | ... | W0_P] (d_in x D).  Rows [o_i, o_{i+1}) belong to adapter
i, which has for every p its own A_ip (d_in x r_ip), B_ip (r_ip x d_p) and
scale s_ip.  For each i and p:
    Z_ip  = X_i A_ip
    Y_i[:, cols_p] = X_i W0_p + s_ip Z_ip B_ip
    dZ_ip = s_ip dY_i[:, cols_p] B_ip^T
    dA_ip = X_i^T dZ_ip
    dB_ip = s_ip Z_ip^T dY_i[:, cols_p]
and the input gradient sums every projection:
    dX_i = sum_p (dY_i[:, cols_p] W0_p^T + dZ_ip A_ip^T)
An adapter with no rows gets zero gradients.  Inputs may be float arrays or,
with dtype="bf16", uint16 bf16 bit patterns; everything is upcast to float64.
"""
from __future__ import annotations

import numpy as np

from .lora import CHUNK, as_f64


def columns(widths):
    """Column offsets c_0 = 0, c_p = d_0 + ... + d_{p-1} of the projections."""
    c = [0]
    for d in widths:
        c.append(c[-1] + int(d))
    return c


def _segments(offsets):
    o = [int(v) for v in offsets]
    return [(o[i], o[i + 1]) for i in range(len(o) - 1)]


def forward_multi(X, W0, A, B, scales, offsets, widths, dtype="fp32", chunk=CHUNK):
    """Y [T, D] and Z[i][p] = X_i A_ip (unscaled), float64.  A, B, scales are
    indexed [adapter][projection]."""
    W = as_f64(W0, dtype)
    cols = columns(widths)
    P = len(widths)
    T = int(offsets[-1])
    Y = np.zeros((T, cols[-1]), dtype=np.float64)
    Z = []
    for i, (a, b) in enumerate(_segments(offsets)):
        Zi = []
        for p in range(P):
            c0, c1 = cols[p], cols[p + 1]
            Aip = as_f64(A[i][p], dtype)
            Bip = as_f64(B[i][p], dtype)
            s = float(scales[i][p])
            Zip = np.zeros((b - a, Aip.shape[1]), dtype=np.float64)
            for r0 in range(a, b, chunk):
                r1 = min(b, r0 + chunk)
                Xc = as_f64(X[r0:r1], dtype)
                Zc = Xc @ Aip
                Y[r0:r1, c0:c1] = Xc @ W[:, c0:c1] + s * (Zc @ Bip)
                Zip[r0 - a:r1 - a] = Zc
            Zi.append(Zip)
        Z.append(Zi)
    return Y, Z


def backward_multi(dY, X, W0, A, B, scales, offsets, widths, dtype="fp32", chunk=CHUNK,
                   want_dx=True):
    """dX [T, d_in] (or None), dA[i][p], dB[i][p], dZ[i][p]."""
    W = as_f64(W0, dtype)
    cols = columns(widths)
    P = len(widths)
    T = int(offsets[-1])
    dX = np.zeros((T, W.shape[0]), dtype=np.float64) if want_dx else None
    dA, dB, dZ = [], [], []
    for i, (a, b) in enumerate(_segments(offsets)):
        gAi, gBi, dZi = [], [], []
        for p in range(P):
            c0, c1 = cols[p], cols[p + 1]
            Aip = as_f64(A[i][p], dtype)
            Bip = as_f64(B[i][p], dtype)
            s = float(scales[i][p])
            gA = np.zeros_like(Aip)
            gB = np.zeros_like(Bip)
            dZip = np.zeros((b - a, Aip.shape[1]), dtype=np.float64)
            for r0 in range(a, b, chunk):
                r1 = min(b, r0 + chunk)
                Xc = as_f64(X[r0:r1], dtype)
                Gp = as_f64(dY[r0:r1], dtype)[:, c0:c1]
                Zc = Xc @ Aip
                dZc = s * (Gp @ Bip.T)
                if want_dx:
                    dX[r0:r1] += Gp @ W[:, c0:c1].T + dZc @ Aip.T
                gA += Xc.T @ dZc
                gB += s * (Zc.T @ Gp)
                dZip[r0 - a:r1 - a] = dZc
            gAi.append(gA)
            gBi.append(gB)
            dZi.append(dZip)
        dA.append(gAi)
        dB.append(gBi)
        dZ.append(dZi)
    return dX, dA, dB, dZ


def sampled_rows_multi(rows, X, W0, A, B, scales, offsets, widths, dY=None, dtype="fp32"):
    """Y, dX and the scaled shrinks s_ip x A_ip on the listed rows only, each
    row from its own adapter as in forward_multi / backward_multi.  Returns
    (Y [len(rows), D], dX [len(rows), d_in] or None, Zs) with Zs[k][p] the
    rank-length vector of row k and projection p."""
    W = as_f64(W0, dtype)
    cols = columns(widths)
    P = len(widths)
    rows = np.asarray(rows, dtype=np.int64)
    own = np.searchsorted(np.asarray(offsets, dtype=np.int64), rows, side="right") - 1
    Y = np.zeros((len(rows), cols[-1]))
    dX = np.zeros((len(rows), W.shape[0])) if dY is not None else None
    Zs = [[None] * P for _ in range(len(rows))]
    for i in np.unique(own):
        ks = np.nonzero(own == i)[0]
        x = as_f64(np.asarray(X)[rows[ks]], dtype)
        g = as_f64(np.asarray(dY)[rows[ks]], dtype) if dY is not None else None
        for p in range(P):
            c0, c1 = cols[p], cols[p + 1]
            Aip = as_f64(A[i][p], dtype)
            Bip = as_f64(B[i][p], dtype)
            s = float(scales[i][p])
            z = s * (x @ Aip)
            Y[ks, c0:c1] = x @ W[:, c0:c1] + z @ Bip
            for q, k in enumerate(ks):
                Zs[k][p] = z[q]
            if g is not None:
                dX[ks] += g[:, c0:c1] @ W[:, c0:c1].T + (s * (g[:, c0:c1] @ Bip.T)) @ Aip.T
    return Y, dX, Zs
