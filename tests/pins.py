"""Checks that pin the oracle to facts other than itself.

Each ``pin_*`` takes the oracle module (``oracle.lora`` or a planted-mistake
copy of it) and raises AssertionError when the oracle disagrees with:
- a hand-worked integer example (tests/golden/hand_example.json);
- the special case B_i = 0, which reduces to a plain matrix product;
- the masked concatenated-rank form of the packed computation (adapters
  concatenated along the rank axis, PLoRA §9.2), computed independently;
- central finite differences of L = sum(dY * Y) (L is affine in every single
  entry of X, A_i, B_i, so the difference quotient is exact up to rounding);
- the merged-weight closed form W0 + s_i A_i B_i (PLoRA §2.1, product read as
  A.B) with a different association order;
- pure-Python triple loops on tiny shapes;
- zero padding of the rank, adapter reordering, linearity in s_i;
- torch CPU float64 autograd of the single-adapter expression;
- for per-token adapter ids: a hand-worked grouping (tests/golden/ids_order.json),
  the definition applied token by token, and the segment form when the ids
  are already in adapter order.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand_case(seed, d_in, d_out, ranks, tokens, scales=None):
    rng = np.random.default_rng(seed)
    n = len(ranks)
    off = np.zeros(n + 1, dtype=np.int64)
    off[1:] = np.cumsum(tokens)
    T = int(off[-1])
    X = rng.standard_normal((T, d_in))
    W0 = rng.standard_normal((d_in, d_out)) * 0.3
    A = [rng.standard_normal((d_in, r)) for r in ranks]
    B = [rng.standard_normal((r, d_out)) for r in ranks]
    dY = rng.standard_normal((T, d_out))
    if scales is None:
        scales = rng.uniform(-2.0, 2.0, size=n)
    return dict(X=X, W0=W0, A=A, B=B, dY=dY, s=np.asarray(scales, dtype=np.float64), off=off)


def _fwd(ol, c):
    return ol.forward(c["X"], c["W0"], c["A"], c["B"], c["s"], c["off"], "fp32", chunk=7)


def _bwd(ol, c):
    return ol.backward(c["dY"], c["X"], c["W0"], c["A"], c["B"], c["s"], c["off"], "fp32", chunk=7)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    den = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) / den if a.size else 0.0
    assert err <= tol, f"{what}: err {err:.3e} > {tol:.1e}"


def pin_hand_example(ol):
    with open(os.path.join(GOLDEN, "hand_example.json")) as f:
        g = json.load(f)
    X = np.asarray(g["X"], dtype=np.float64)
    W0 = np.asarray(g["W0"], dtype=np.float64)
    A = [np.asarray(a, dtype=np.float64) for a in g["A"]]
    B = [np.asarray(b, dtype=np.float64) for b in g["B"]]
    dY = np.asarray(g["dY"], dtype=np.float64)
    s = np.asarray(g["scales"])
    off = np.asarray(g["offsets"])
    e = g["expect"]
    Y, Z = ol.forward(X, W0, A, B, s, off, "fp32")
    assert np.array_equal(Y, np.asarray(e["Y"], dtype=np.float64)), Y
    for i in range(len(A)):
        assert np.array_equal(Z[i].reshape(-1), np.asarray(e["Z"][i], dtype=np.float64).reshape(-1))
    dX, dA, dB, dZ = ol.backward(dY, X, W0, A, B, s, off, "fp32")
    assert np.array_equal(dX, np.asarray(e["dX"], dtype=np.float64)), dX
    for i in range(len(A)):
        assert np.array_equal(dA[i], np.asarray(e["dA"][i], dtype=np.float64)), (i, dA[i])
        assert np.array_equal(dB[i], np.asarray(e["dB"][i], dtype=np.float64)), (i, dB[i])
        assert np.array_equal(dZ[i].reshape(-1), np.asarray(e["dZ"][i], dtype=np.float64).reshape(-1))


def pin_b_zero(ol):
    c = rand_case(1, 12, 10, [3, 5, 2], [9, 0, 14])
    c["B"] = [np.zeros_like(b) for b in c["B"]]
    Y, Z = _fwd(ol, c)
    _close(Y, c["X"] @ c["W0"], 1e-13, "Y with B=0")
    dX, dA, dB, dZ = _bwd(ol, c)
    _close(dX, c["dY"] @ c["W0"].T, 1e-13, "dX with B=0")
    for i in range(3):
        assert np.all(dA[i] == 0.0), "dA must vanish when B=0"
        assert np.all(dZ[i] == 0.0)
    # dB_i = s_i (X_i A_i)^T dY_i  by a single product over the segment
    o = c["off"]
    for i in range(3):
        Xi = c["X"][o[i]:o[i + 1]]
        ref = c["s"][i] * ((Xi @ c["A"][i]).T @ c["dY"][o[i]:o[i + 1]])
        _close(dB[i], ref, 1e-13, "dB with B=0")


def fused_concat_form(c):
    """Packed computation as one product over the concatenated rank axis:
    Z_full = X A_cat; each row keeps only its own adapter's rank columns
    (times s_i), then Y = X W0 + Z_masked B_cat.  Backward by the same mask."""
    X, W0, dY = c["X"], c["W0"], c["dY"]
    ranks = [a.shape[1] for a in c["A"]]
    A_cat = np.concatenate(c["A"], axis=1)
    B_cat = np.concatenate(c["B"], axis=0)
    R = sum(ranks)
    T = X.shape[0]
    mask = np.zeros((T, R))
    col = 0
    o = c["off"]
    for i, r in enumerate(ranks):
        mask[o[i]:o[i + 1], col:col + r] = c["s"][i]
        col += r
    Zf = X @ A_cat
    Y = X @ W0 + (Zf * mask) @ B_cat
    dZf = (dY @ B_cat.T) * mask
    dX = dY @ W0.T + dZf @ A_cat.T
    dA_cat = X.T @ dZf
    dB_cat = (Zf * mask).T @ dY
    dA, dB = [], []
    col = 0
    for r in ranks:
        dA.append(dA_cat[:, col:col + r])
        dB.append(dB_cat[col:col + r])
        col += r
    return Y, dX, dA, dB


def pin_fused_equals_sequential(ol):
    c = rand_case(2, 16, 11, [4, 1, 7, 3], [5, 13, 0, 21])
    Y, _ = _fwd(ol, c)
    dX, dA, dB, _ = _bwd(ol, c)
    Yf, dXf, dAf, dBf = fused_concat_form(c)
    _close(Y, Yf, 1e-12, "Y fused")
    _close(dX, dXf, 1e-12, "dX fused")
    for i in range(4):
        _close(dA[i], dAf[i], 1e-12, "dA fused")
        _close(dB[i], dBf[i], 1e-12, "dB fused")


def pin_finite_differences(ol):
    c = rand_case(3, 9, 7, [3, 2], [6, 5])
    dX, dA, dB, _ = _bwd(ol, c)
    rng = np.random.default_rng(33)

    def loss(cc):
        Y, _ = _fwd(ol, cc)
        return float(np.sum(cc["dY"] * Y))

    h = 1e-3
    for _ in range(12):
        t, j = rng.integers(0, 11), rng.integers(0, 9)
        cp, cm = dict(c), dict(c)
        cp["X"] = c["X"].copy(); cp["X"][t, j] += h
        cm["X"] = c["X"].copy(); cm["X"][t, j] -= h
        fd = (loss(cp) - loss(cm)) / (2 * h)
        assert abs(fd - dX[t, j]) <= 1e-8 * max(1.0, abs(fd)), ("dX", fd, dX[t, j])
    for i in range(2):
        for _ in range(8):
            p, q = rng.integers(0, c["A"][i].shape[0]), rng.integers(0, c["A"][i].shape[1])
            cp, cm = dict(c), dict(c)
            cp["A"] = [a.copy() for a in c["A"]]; cp["A"][i][p, q] += h
            cm["A"] = [a.copy() for a in c["A"]]; cm["A"][i][p, q] -= h
            fd = (loss(cp) - loss(cm)) / (2 * h)
            assert abs(fd - dA[i][p, q]) <= 1e-8 * max(1.0, abs(fd)), ("dA", i, fd, dA[i][p, q])
            p, q = rng.integers(0, c["B"][i].shape[0]), rng.integers(0, c["B"][i].shape[1])
            cp, cm = dict(c), dict(c)
            cp["B"] = [b.copy() for b in c["B"]]; cp["B"][i][p, q] += h
            cm["B"] = [b.copy() for b in c["B"]]; cm["B"][i][p, q] -= h
            fd = (loss(cp) - loss(cm)) / (2 * h)
            assert abs(fd - dB[i][p, q]) <= 1e-8 * max(1.0, abs(fd)), ("dB", i, fd, dB[i][p, q])


def pin_merged_weight(ol):
    c = rand_case(4, 10, 13, [2, 6, 3], [7, 4, 12])
    Y, _ = _fwd(ol, c)
    dX, dA, dB, _ = _bwd(ol, c)
    o = c["off"]
    for i in range(3):
        s = c["s"][i]
        Wm = c["W0"] + s * (c["A"][i] @ c["B"][i])
        Xi, dYi = c["X"][o[i]:o[i + 1]], c["dY"][o[i]:o[i + 1]]
        _close(Y[o[i]:o[i + 1]], Xi @ Wm, 1e-12, "Y merged")
        _close(dX[o[i]:o[i + 1]], dYi @ Wm.T, 1e-12, "dX merged")
        G = Xi.T @ dYi
        _close(dA[i], s * (G @ c["B"][i].T), 1e-12, "dA merged")
        _close(dB[i], s * (c["A"][i].T @ G), 1e-12, "dB merged")


def pin_brute_force(ol):
    c = rand_case(5, 5, 4, [2, 3], [3, 4])
    Y, _ = _fwd(ol, c)
    dX, dA, dB, _ = _bwd(ol, c)
    X, W0, dY, o = c["X"].tolist(), c["W0"].tolist(), c["dY"].tolist(), c["off"].tolist()
    d_in, d_out = 5, 4
    for i in range(2):
        A, B, s = c["A"][i].tolist(), c["B"][i].tolist(), float(c["s"][i])
        r = len(B)
        gA = [[0.0] * r for _ in range(d_in)]
        gB = [[0.0] * d_out for _ in range(r)]
        for t in range(o[i], o[i + 1]):
            z = [sum(X[t][k] * A[k][q] for k in range(d_in)) for q in range(r)]
            for j in range(d_out):
                y = sum(X[t][k] * W0[k][j] for k in range(d_in)) + s * sum(z[q] * B[q][j] for q in range(r))
                assert abs(y - Y[t, j]) <= 1e-13 * max(1.0, abs(y)), ("Y", t, j)
            dz = [s * sum(dY[t][j] * B[q][j] for j in range(d_out)) for q in range(r)]
            for k in range(d_in):
                dx = sum(dY[t][j] * W0[k][j] for j in range(d_out)) + sum(dz[q] * A[k][q] for q in range(r))
                assert abs(dx - dX[t, k]) <= 1e-13 * max(1.0, abs(dx)), ("dX", t, k)
                for q in range(r):
                    gA[k][q] += X[t][k] * dz[q]
            for q in range(r):
                for j in range(d_out):
                    gB[q][j] += s * z[q] * dY[t][j]
        _close(dA[i], np.asarray(gA), 1e-13, "dA brute")
        _close(dB[i], np.asarray(gB), 1e-13, "dB brute")


def pin_rank_padding(ol):
    c = rand_case(6, 8, 9, [3, 5], [6, 7])
    Y, _ = _fwd(ol, c)
    dX, dA, dB, _ = _bwd(ol, c)
    p = dict(c)
    p["A"] = [np.concatenate([a, np.zeros((a.shape[0], 4))], axis=1) for a in c["A"]]
    p["B"] = [np.concatenate([b, np.zeros((4, b.shape[1]))], axis=0) for b in c["B"]]
    Yp, _ = _fwd(ol, p)
    dXp, dAp, dBp, _ = _bwd(ol, p)
    _close(Yp, Y, 1e-13, "Y padded")
    _close(dXp, dX, 1e-13, "dX padded")
    for i, r in enumerate([3, 5]):
        _close(dAp[i][:, :r], dA[i], 1e-13, "dA padded")
        _close(dBp[i][:r], dB[i], 1e-13, "dB padded")
        assert np.all(dAp[i][:, r:] == 0.0) and np.all(dBp[i][r:] == 0.0)


def pin_permutation(ol):
    c = rand_case(7, 6, 5, [2, 4, 3], [4, 6, 5])
    Y, _ = _fwd(ol, c)
    dX, dA, dB, _ = _bwd(ol, c)
    perm = [2, 0, 1]
    o = c["off"]
    rows = np.concatenate([np.arange(o[i], o[i + 1]) for i in perm])
    q = dict(c)
    q["X"], q["dY"] = c["X"][rows], c["dY"][rows]
    q["A"] = [c["A"][i] for i in perm]
    q["B"] = [c["B"][i] for i in perm]
    q["s"] = c["s"][perm]
    toks = [int(o[i + 1] - o[i]) for i in perm]
    q["off"] = np.concatenate([[0], np.cumsum(toks)]).astype(np.int64)
    Yq, _ = _fwd(ol, q)
    dXq, dAq, dBq, _ = _bwd(ol, q)
    _close(Yq, Y[rows], 1e-12, "Y permuted")
    _close(dXq, dX[rows], 1e-12, "dX permuted")
    for k, i in enumerate(perm):
        _close(dAq[k], dA[i], 1e-12, "dA permuted")
        _close(dBq[k], dB[i], 1e-12, "dB permuted")


def pin_scale_linearity(ol):
    c = rand_case(8, 7, 6, [3, 2], [5, 8])
    base_Y = c["X"] @ c["W0"]
    base_dX = c["dY"] @ c["W0"].T
    z = dict(c); z["s"] = np.zeros(2)
    Y0, _ = _fwd(ol, z)
    dX0, dA0, dB0, _ = _bwd(ol, z)
    _close(Y0, base_Y, 1e-13, "Y at s=0")
    _close(dX0, base_dX, 1e-13, "dX at s=0")
    assert all(np.all(a == 0) for a in dA0) and all(np.all(b == 0) for b in dB0)
    Y1, _ = _fwd(ol, c)
    dX1, dA1, dB1, _ = _bwd(ol, c)
    d = dict(c); d["s"] = 2 * c["s"]
    Y2, _ = _fwd(ol, d)
    dX2, dA2, dB2, _ = _bwd(ol, d)
    _close(Y2 - base_Y, 2 * (Y1 - base_Y), 1e-13, "Y linear in s")
    _close(dX2 - base_dX, 2 * (dX1 - base_dX), 1e-13, "dX linear in s")
    for i in range(2):
        _close(dA2[i], 2 * dA1[i], 1e-13, "dA linear in s")
        _close(dB2[i], 2 * dB1[i], 1e-13, "dB linear in s")


def pin_torch_autograd(ol):
    import torch
    c = rand_case(9, 12, 10, [4, 2], [7, 9])
    Y, _ = _fwd(ol, c)
    dX, dA, dB, _ = _bwd(ol, c)
    o = c["off"]
    for i in range(2):
        Xi = torch.tensor(c["X"][o[i]:o[i + 1]], requires_grad=True)
        Ai = torch.tensor(c["A"][i], requires_grad=True)
        Bi = torch.tensor(c["B"][i], requires_grad=True)
        W = torch.tensor(c["W0"])
        Yi = Xi @ W + float(c["s"][i]) * ((Xi @ Ai) @ Bi)
        Yi.backward(torch.tensor(c["dY"][o[i]:o[i + 1]]))
        _close(Y[o[i]:o[i + 1]], Yi.detach().numpy(), 1e-12, "Y torch")
        _close(dX[o[i]:o[i + 1]], Xi.grad.numpy(), 1e-12, "dX torch")
        _close(dA[i], Ai.grad.numpy(), 1e-12, "dA torch")
        _close(dB[i], Bi.grad.numpy(), 1e-12, "dB torch")


def pin_sampled_rows(ol):
    c = rand_case(10, 9, 8, [3, 1, 2], [4, 0, 9])
    Y, _ = _fwd(ol, c)
    dX, _, _, _ = _bwd(ol, c)
    rows = [0, 3, 4, 12]
    Ys, dXs = ol.sampled_rows(rows, c["X"], c["W0"], c["A"], c["B"], c["s"], c["off"], dY=c["dY"])
    _close(Ys, Y[rows], 1e-13, "sampled Y")
    _close(dXs, dX[rows], 1e-13, "sampled dX")


def pin_sampled_z_rows(ol):
    # the scaled shrink of each sampled row equals the saved activation the
    # full forward returns for that row
    c = rand_case(10, 9, 8, [3, 1, 2], [4, 0, 9])
    _, Zs = _fwd(ol, c)
    rows = [0, 3, 4, 12]
    _, _, zr = ol.sampled_rows(rows, c["X"], c["W0"], c["A"], c["B"], c["s"], c["off"], with_z=True)
    own = ol.adapter_of_rows(c["off"], rows)
    for k, (t, i) in enumerate(zip(rows, own)):
        _close(zr[k], float(c["s"][i]) * Zs[i][t - c["off"][i]], 1e-13, "sampled Z")


def pin_bf16_decode(ol):
    # bf16 bit patterns: 0x3F80 = 1.0, 0xC000 = -2.0, 0x3E80 = 0.25, 0x0000 = 0.
    bits = np.asarray([[0x3F80, 0xC000], [0x3E80, 0x0000]], dtype=np.uint16)
    assert np.array_equal(ol.as_f64(bits, "bf16"), np.asarray([[1.0, -2.0], [0.25, 0.0]]))


def pin_ids_golden_order(ol):
    """Grouping per-token ids, worked by hand (tests/golden/ids_order.json)."""
    with open(os.path.join(GOLDEN, "ids_order.json")) as f:
        g = json.load(f)
    perm, off = ol.ids_order(g["token_adapter"], g["n"])
    assert [int(v) for v in perm] == g["perm"], perm
    assert [int(v) for v in off] == g["offsets"], off


def pin_ids_brute_force(ol):
    """Per-token ids against the definition applied token by token on tiny
    shapes: each row uses its own adapter; each adapter's gradients sum over
    its tokens (pure-Python loops over tokens, outer products per token)."""
    rng = np.random.default_rng(23)
    n, d_in, d_out, T = 3, 5, 4, 11
    ranks = [2, 1, 3]
    ids = rng.integers(0, n, size=T)
    ids[3] = 2  # every adapter present ...
    ids[7] = 0
    ids[9] = 1
    X = rng.standard_normal((T, d_in))
    dY = rng.standard_normal((T, d_out))
    W0 = rng.standard_normal((d_in, d_out))
    A = [rng.standard_normal((d_in, r)) for r in ranks]
    B = [rng.standard_normal((r, d_out)) for r in ranks]
    s = np.array([0.5, -1.5, 2.0])
    Y_ref = np.zeros((T, d_out))
    dX_ref = np.zeros((T, d_in))
    dA_ref = [np.zeros_like(a) for a in A]
    dB_ref = [np.zeros_like(b) for b in B]
    for t in range(T):
        a = int(ids[t])
        z = X[t] @ A[a]
        Y_ref[t] = X[t] @ W0 + s[a] * (z @ B[a])
        dz = s[a] * (B[a] @ dY[t])
        dX_ref[t] = W0 @ dY[t] + A[a] @ dz
        dA_ref[a] += np.outer(X[t], dz)
        dB_ref[a] += s[a] * np.outer(z, dY[t])
    Y, _ = ol.forward_ids(X, W0, A, B, s, ids, "fp32", chunk=2)
    dX, dA, dB, _ = ol.backward_ids(dY, X, W0, A, B, s, ids, "fp32", chunk=2)
    _close(Y, Y_ref, 1e-12, "Y ids")
    _close(dX, dX_ref, 1e-12, "dX ids")
    for i in range(n):
        _close(dA[i], dA_ref[i], 1e-12, f"dA{i} ids")
        _close(dB[i], dB_ref[i], 1e-12, f"dB{i} ids")


def pin_ids_sorted_is_segments(ol):
    """Ids already in adapter order give exactly the segment form."""
    c = rand_case(29, 6, 5, [2, 4], [3, 5])
    ids = np.repeat([0, 1], [3, 5])
    Y, _ = ol.forward_ids(c["X"], c["W0"], c["A"], c["B"], c["s"], ids, "fp32", chunk=7)
    Ys, _ = _fwd(ol, c)
    assert np.array_equal(Y, Ys)
    dX, dA, dB, _ = ol.backward_ids(c["dY"], c["X"], c["W0"], c["A"], c["B"], c["s"], ids, "fp32", chunk=7)
    dXs, dAs, dBs, _ = _bwd(ol, c)
    assert np.array_equal(dX, dXs)
    for i in range(2):
        assert np.array_equal(dA[i], dAs[i]) and np.array_equal(dB[i], dBs[i])


ALL_PINS = [pin_ids_golden_order, pin_ids_brute_force, pin_ids_sorted_is_segments, pin_hand_example, pin_b_zero, pin_fused_equals_sequential, pin_finite_differences,
            pin_merged_weight, pin_brute_force, pin_rank_padding, pin_permutation,
            pin_scale_linearity, pin_torch_autograd, pin_sampled_rows, pin_sampled_z_rows,
            pin_bf16_decode]
