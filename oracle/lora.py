"""Per-adapter LoRA forward/backward in float64 -- TEST INFRASTRUCTURE ONLY.

Parity pinned: see tests/test_oracle_pins.py (closed forms, invariants,
finite differences, brute force, torch autograd, a hand-computed example).

Definition followed (PLoRA: Efficient Concurrent LoRA Training for Large
Language Models):
- §2.1: a frozen W of shape (d, k); trainable A of shape (d, r) and B of shape
  (r, k); the update is the product of the two with a scaling factor.  The page
  prints the product as "B x A", which the stated shapes do not allow; the
  product that fits them is A.B (d x k), and that is what is used.
- §2.4: every packed adapter computes exactly what standard LoRA fine-tuning
  computes on its own inputs; the base is shared.
- §9.2: adapters are concatenated; the token axis is sequence length times
  batch size; the backward produces dB (Case 1), the gradient into B's input
  (Case 2), dA (Case 3) and the gradient into A's input (Case 4).

Rows [o_i, o_{i+1}) of the packed token axis belong to adapter i.  For each i:
    Z_i  = X_i A_i
    Y_i  = X_i W0 + s_i Z_i B_i
    dZ_i = s_i dY_i B_i^T
    dX_i = dY_i W0^T + dZ_i A_i^T
    dA_i = X_i^T dZ_i
    dB_i = s_i Z_i^T dY_i
An adapter with no rows gets dA_i = 0 and dB_i = 0.  W0 gets no gradient.

With per-token adapter ids instead of segments (forward_ids, backward_ids),
the same is computed over the rows of each adapter, with row-indexed results
in the caller's row order.

Inputs may be float arrays or, with ``dtype="bf16"``, uint16 arrays holding
bf16 bit patterns; everything is upcast to float64 and no intermediate
rounding is modelled.  Work streams over row chunks so large inputs need not
be held in float64 all at once.
"""
from __future__ import annotations

import numpy as np

CHUNK = 4096


def as_f64(a, dtype: str) -> np.ndarray:
    """Upcast an input array to float64 (bf16 given as uint16 bit patterns)."""
    a = np.asarray(a)
    if dtype == "bf16":
        assert a.dtype == np.uint16
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _segments(offsets):
    o = [int(v) for v in offsets]
    return [(o[i], o[i + 1]) for i in range(len(o) - 1)]


def forward(X, W0, A, B, scales, offsets, dtype="fp32", chunk=CHUNK):
    """Y [T, d_out] and Z_i = X_i A_i (unscaled) for every adapter, float64."""
    W = as_f64(W0, dtype)
    T = int(offsets[-1])
    Y = np.zeros((T, W.shape[1]), dtype=np.float64)
    Z = []
    for i, (a, b) in enumerate(_segments(offsets)):
        Ai = as_f64(A[i], dtype)
        Bi = as_f64(B[i], dtype)
        s = float(scales[i])
        Zi = np.zeros((b - a, Ai.shape[1]), dtype=np.float64)
        for r0 in range(a, b, chunk):
            r1 = min(b, r0 + chunk)
            Xc = as_f64(X[r0:r1], dtype)
            Zc = Xc @ Ai
            Y[r0:r1] = Xc @ W + s * (Zc @ Bi)
            Zi[r0 - a:r1 - a] = Zc
        Z.append(Zi)
    return Y, Z


def backward(dY, X, W0, A, B, scales, offsets, dtype="fp32", chunk=CHUNK, want_dx=True):
    """dX [T, d_in] (or None), dA_i [d_in, r_i], dB_i [r_i, d_out], dZ_i = s_i dY_i B_i^T."""
    W = as_f64(W0, dtype)
    T = int(offsets[-1])
    dX = np.zeros((T, W.shape[0]), dtype=np.float64) if want_dx else None
    dA, dB, dZ = [], [], []
    for i, (a, b) in enumerate(_segments(offsets)):
        Ai = as_f64(A[i], dtype)
        Bi = as_f64(B[i], dtype)
        s = float(scales[i])
        gA = np.zeros_like(Ai)
        gB = np.zeros_like(Bi)
        dZi = np.zeros((b - a, Ai.shape[1]), dtype=np.float64)
        for r0 in range(a, b, chunk):
            r1 = min(b, r0 + chunk)
            Xc = as_f64(X[r0:r1], dtype)
            dYc = as_f64(dY[r0:r1], dtype)
            Zc = Xc @ Ai
            dZc = s * (dYc @ Bi.T)
            if want_dx:
                dX[r0:r1] = dYc @ W.T + dZc @ Ai.T
            gA += Xc.T @ dZc
            gB += s * (Zc.T @ dYc)
            dZi[r0 - a:r1 - a] = dZc
        dA.append(gA)
        dB.append(gB)
        dZ.append(dZi)
    return dX, dA, dB, dZ


def ids_order(token_adapter, n):
    """Rows grouped by adapter for per-token adapter ids: token t belongs to
    adapter token_adapter[t] (0 <= id < n); each adapter's rows keep the
    caller's order (a stable sort by id).  Returns (perm, offsets): grouped
    row i is the caller's row perm[i], and adapter a owns grouped rows
    [offsets[a], offsets[a+1])."""
    ids = np.asarray(token_adapter, dtype=np.int64)
    assert ids.ndim == 1 and (ids.size == 0 or (ids.min() >= 0 and ids.max() < n))
    perm = np.argsort(ids, kind="stable")
    offsets = np.zeros(n + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(np.bincount(ids, minlength=n))
    return perm, offsets


def forward_ids(X, W0, A, B, scales, token_adapter, dtype="fp32", chunk=CHUNK):
    """forward() for rows in the caller's order with per-token adapter ids:
    Y in the caller's row order; Z_i over adapter i's rows in that order."""
    perm, off = ids_order(token_adapter, len(A))
    Yg, Z = forward(np.asarray(X)[perm], W0, A, B, scales, off, dtype, chunk)
    Y = np.empty_like(Yg)
    Y[perm] = Yg
    return Y, Z


def backward_ids(dY, X, W0, A, B, scales, token_adapter, dtype="fp32", chunk=CHUNK, want_dx=True):
    """backward() for rows in the caller's order with per-token adapter ids:
    dX in the caller's row order."""
    perm, off = ids_order(token_adapter, len(A))
    dXg, dA, dB, dZ = backward(np.asarray(dY)[perm], np.asarray(X)[perm], W0, A, B, scales, off, dtype,
                               chunk, want_dx)
    dX = None
    if want_dx:
        dX = np.empty_like(dXg)
        dX[perm] = dXg
    return dX, dA, dB, dZ


def adapter_of_rows(offsets, rows):
    """Adapter index owning each packed row."""
    o = np.asarray(offsets, dtype=np.int64)
    return np.searchsorted(o, np.asarray(rows, dtype=np.int64), side="right") - 1


def sampled_rows(rows, X, W0, A, B, scales, offsets, dY=None, dtype="fp32", with_z=False):
    """Y (and dX if dY is given) on the listed packed rows only, float64.

    Each row is computed from its own adapter exactly as in ``forward`` /
    ``backward``; used to check full-size outputs one row at a time.  With
    ``with_z`` the scaled shrink s_i * x A_i of each row is returned as a
    third value (a list of rank-length vectors)."""
    W = as_f64(W0, dtype)
    rows = np.asarray(rows, dtype=np.int64)
    own = adapter_of_rows(offsets, rows)
    Y = np.zeros((len(rows), W.shape[1]))
    dX = np.zeros((len(rows), W.shape[0])) if dY is not None else None
    Zs = [None] * len(rows)
    # rows of one adapter are stacked so each product is one matrix product
    for i in np.unique(own):
        ks = np.nonzero(own == i)[0]
        Ai = as_f64(A[i], dtype)
        Bi = as_f64(B[i], dtype)
        s = float(scales[i])
        x = as_f64(np.asarray(X)[rows[ks]], dtype)
        Y[ks] = x @ W + s * ((x @ Ai) @ Bi)
        if with_z:
            zi = s * (x @ Ai)
            for q, k in enumerate(ks):
                Zs[k] = zi[q]
        if dY is not None:
            g = as_f64(np.asarray(dY)[rows[ks]], dtype)
            dX[ks] = g @ W.T + (s * (g @ Bi.T)) @ Ai.T
    if with_z:
        return Y, dX, Zs
    return Y, dX


def max_rel_err(got, ref) -> float:
    """Normwise-max relative error max|g - o| / max|o|.  With max|o| = 0 the
    result is 0 if g is all zero and +inf otherwise."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(ref)))
    num = float(np.max(np.abs(got - ref)))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den
