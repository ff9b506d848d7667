"""Checks that pin the multi-projection oracle (oracle/multi.py) to facts
other than itself.

Each ``pin_*`` takes the module (or a planted-mistake copy) and raises when
it disagrees with:
- the single-projection oracle (itself pinned in tests/pins.py) when there is
  one projection;
- independent packed layers, one per projection, run through the
  single-projection oracle on the projection's columns of W0 and dY, with dX
  their sum;
- torch float64 autograd of the block-diagonal form: per adapter,
  Y_i = X_i W0 + (X_i [A_i1 .. A_iP]) blockdiag(s_i1 B_i1, .., s_iP B_iP),
  differentiated through L = sum(dY * Y);
- pure-Python loops on tiny shapes;
- the sampled-row form against the whole results.
"""
from __future__ import annotations

import numpy as np

from oracle import lora as ol


def _case(seed, d_in, widths, ranks, tokens):
    rng = np.random.default_rng(seed)
    n, P = len(tokens), len(widths)
    off = np.zeros(n + 1, dtype=np.int64)
    off[1:] = np.cumsum(tokens)
    T = int(off[-1])
    D = int(sum(widths))
    X = rng.standard_normal((T, d_in))
    W0 = rng.standard_normal((d_in, D)) * 0.3
    A = [[rng.standard_normal((d_in, ranks[i][p])) for p in range(P)] for i in range(n)]
    B = [[rng.standard_normal((ranks[i][p], widths[p])) for p in range(P)] for i in range(n)]
    s = [[float(rng.uniform(-2, 2)) for _ in range(P)] for _ in range(n)]
    dY = rng.standard_normal((T, D))
    return dict(X=X, W0=W0, A=A, B=B, s=s, off=off, dY=dY, widths=list(widths))


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    den = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) / den if a.size else 0.0
    assert err <= tol, f"{what}: err {err:.3e} > {tol:.1e}"


def _run(om, c, chunk=5):
    Y, Z = om.forward_multi(c["X"], c["W0"], c["A"], c["B"], c["s"], c["off"], c["widths"], chunk=chunk)
    dX, dA, dB, dZ = om.backward_multi(c["dY"], c["X"], c["W0"], c["A"], c["B"], c["s"], c["off"],
                                       c["widths"], chunk=chunk)
    return Y, Z, dX, dA, dB, dZ


def pin_multi_one_projection(om):
    c = _case(1, 12, [10], [[3], [1], [5]], [7, 0, 9])
    Y, Z, dX, dA, dB, _ = _run(om, c)
    A1 = [a[0] for a in c["A"]]
    B1 = [b[0] for b in c["B"]]
    s1 = [v[0] for v in c["s"]]
    Yr, Zr = ol.forward(c["X"], c["W0"], A1, B1, s1, c["off"])
    dXr, dAr, dBr, _ = ol.backward(c["dY"], c["X"], c["W0"], A1, B1, s1, c["off"])
    _close(Y, Yr, 1e-12, "Y")
    _close(dX, dXr, 1e-12, "dX")
    for i in range(3):
        _close(Z[i][0], Zr[i], 1e-12, f"Z{i}")
        _close(dA[i][0], dAr[i], 1e-12, f"dA{i}")
        _close(dB[i][0], dBr[i], 1e-12, f"dB{i}")


def pin_multi_equals_per_projection_layers(om):
    widths = [8, 4, 4]
    c = _case(2, 16, widths, [[2, 3, 1], [4, 4, 4], [1, 6, 2], [3, 1, 5]], [5, 11, 0, 6])
    Y, Z, dX, dA, dB, _ = _run(om, c)
    cols = [0, 8, 12, 16]
    dX_sum = np.zeros_like(c["X"])
    for p in range(3):
        Wp = c["W0"][:, cols[p]:cols[p + 1]]
        Ap = [a[p] for a in c["A"]]
        Bp = [b[p] for b in c["B"]]
        sp = [v[p] for v in c["s"]]
        Yp, Zp = ol.forward(c["X"], Wp, Ap, Bp, sp, c["off"])
        dXp, dAp, dBp, _ = ol.backward(np.ascontiguousarray(c["dY"][:, cols[p]:cols[p + 1]]), c["X"], Wp,
                                       Ap, Bp, sp, c["off"])
        _close(Y[:, cols[p]:cols[p + 1]], Yp, 1e-12, f"Y projection {p}")
        dX_sum += dXp
        for i in range(4):
            _close(Z[i][p], Zp[i], 1e-12, f"Z {i},{p}")
            _close(dA[i][p], dAp[i], 1e-12, f"dA {i},{p}")
            _close(dB[i][p], dBp[i], 1e-12, f"dB {i},{p}")
    _close(dX, dX_sum, 1e-12, "dX is the sum over projections")


def pin_multi_torch_block_diagonal(om):
    import torch
    widths = [6, 3]
    ranks = [[2, 3], [4, 1], [1, 1]]
    c = _case(3, 10, widths, ranks, [4, 6, 3])
    Y, Z, dX, dA, dB, _ = _run(om, c)
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    X = t(c["X"])
    W0 = torch.tensor(c["W0"], dtype=torch.float64)
    A = [[t(a) for a in ai] for ai in c["A"]]
    B = [[t(b) for b in bi] for bi in c["B"]]
    outs = []
    for i, (lo, hi) in enumerate(zip(c["off"][:-1], c["off"][1:])):
        Acat = torch.cat(A[i], dim=1)
        Bdiag = torch.block_diag(*[c["s"][i][p] * B[i][p] for p in range(2)])
        outs.append(X[lo:hi] @ W0 + (X[lo:hi] @ Acat) @ Bdiag)
    Yt = torch.cat(outs, dim=0)
    L = (Yt * torch.tensor(c["dY"])).sum()
    L.backward()
    _close(Y, Yt.detach().numpy(), 1e-12, "Y vs torch")
    _close(dX, X.grad.numpy(), 1e-12, "dX vs torch")
    for i in range(3):
        for p in range(2):
            _close(dA[i][p], A[i][p].grad.numpy(), 1e-12, f"dA {i},{p} vs torch")
            _close(dB[i][p], B[i][p].grad.numpy(), 1e-12, f"dB {i},{p} vs torch")


def pin_multi_brute_force(om):
    widths = [2, 3]
    ranks = [[1, 2], [2, 1]]
    c = _case(4, 3, widths, ranks, [2, 3])
    Y, Z, dX, dA, dB, _ = _run(om, c, chunk=1)
    X, W0, dY = c["X"], c["W0"], c["dY"]
    cols = [0, 2, 5]
    seg = [0, 0, 1, 1, 1]
    for t in range(5):
        i = seg[t]
        for p in range(2):
            Ap, Bp, s = c["A"][i][p], c["B"][i][p], c["s"][i][p]
            for o in range(cols[p], cols[p + 1]):
                v = sum(X[t][k] * W0[k][o] for k in range(3))
                for q in range(ranks[i][p]):
                    z = sum(X[t][k] * Ap[k][q] for k in range(3))
                    v += s * z * Bp[q][o - cols[p]]
                assert abs(v - Y[t][o]) < 1e-12, ("Y", t, o)
        for k in range(3):
            g = sum(dY[t][o] * W0[k][o] for o in range(5))
            for p in range(2):
                Ap, Bp, s = c["A"][i][p], c["B"][i][p], c["s"][i][p]
                for q in range(ranks[i][p]):
                    dz = s * sum(dY[t][o] * Bp[q][o - cols[p]] for o in range(cols[p], cols[p + 1]))
                    g += dz * Ap[k][q]
            assert abs(g - dX[t][k]) < 1e-12, ("dX", t, k)
    for i, rows in ((0, [0, 1]), (1, [2, 3, 4])):
        for p in range(2):
            Ap, Bp, s = c["A"][i][p], c["B"][i][p], c["s"][i][p]
            for q in range(ranks[i][p]):
                for k in range(3):
                    ga = sum(X[t][k] * s * sum(dY[t][o] * Bp[q][o - cols[p]] for o in range(cols[p], cols[p + 1]))
                             for t in rows)
                    assert abs(ga - dA[i][p][k][q]) < 1e-12, ("dA", i, p, k, q)
                for o in range(cols[p], cols[p + 1]):
                    gb = sum(s * sum(X[t][k] * Ap[k][q] for k in range(3)) * dY[t][o] for t in rows)
                    assert abs(gb - dB[i][p][q][o - cols[p]]) < 1e-12, ("dB", i, p, q, o)


def pin_multi_sampled(om):
    widths = [4, 8]
    ranks = [[2, 1], [3, 5], [1, 2]]
    c = _case(5, 12, widths, ranks, [6, 0, 9])
    Y, Z, dX, dA, dB, _ = _run(om, c)
    rows = [0, 5, 6, 14]
    Ys, dXs, Zs = om.sampled_rows_multi(rows, c["X"], c["W0"], c["A"], c["B"], c["s"], c["off"], widths,
                                        dY=c["dY"])
    _close(Ys, Y[rows], 1e-12, "sampled Y")
    _close(dXs, dX[rows], 1e-12, "sampled dX")
    own = [0, 0, 2, 2]
    for k, t in enumerate(rows):
        i = own[k]
        for p in range(2):
            _close(Zs[k][p], c["s"][i][p] * Z[i][p][t - c["off"][i]], 1e-12, f"sampled Z row {t}")


ALL_PINS = [pin_multi_one_projection, pin_multi_equals_per_projection_layers, pin_multi_torch_block_diagonal,
            pin_multi_brute_force, pin_multi_sampled]
