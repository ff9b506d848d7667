"""Seeded sweep of layer configurations on the GPU against the oracles.

Each case draws (from its own seed) a dtype, a W0 layout, a stream count,
1-8 adapters with ranks 1-256 and token counts 0-700 (empty and ragged
segments), dimensions that are multiples of 64 (from 64 to 1536, so that
some GEMM launches split K and some do not), and one of five plan kinds:
segments, per-token ids in a shuffled order, several projections sharing
the input (with segments or with shuffled ids), or a microscaled base
(MXFP8 and MXFP4 in turn); about one case in seven holds the base in both
layouts.  Every output is compared with the oracle at
the dtype's bar: Y, dX, every dA_i and dB_i, and the saved activation Z'
(padding columns exactly zero)."""
import numpy as np
import pytest

from oracle import lora as ol
from oracle import multi as om
from oracle import mx as omx
from tests.gpu_harness import TOL, custom_workload, say, to_dev, to_host_f64
from workloads.multi import host_multi
from workloads.mx import pack, quantize_mx, quantize_mx4
from workloads.tensors import host_tensors

N_CASES = 240


def draw_case(seed):
    g = np.random.default_rng(1000 + seed)
    kind = ["segments", "ids", "multi", "mxfp8", "multi_ids"][seed % 5]
    dt = "fp32" if (kind != "mxfp8" and g.random() < 0.3) else "bf16"
    n = int(g.integers(1, 9))
    ranks = [int(g.choice([1, 4, 8, 16, 31, 33, 64, 100, 128, 200, 256])) for _ in range(n)]
    tokens = [int(g.choice([0, 1, 17, int(g.integers(1, 700))])) for _ in range(n)]
    if sum(tokens) == 0:
        tokens[0] = 33
    d_in = 64 * int(g.integers(1, 25))
    d_out = 64 * int(g.integers(1, 25))
    layout = "nk" if g.random() < 0.4 else "kn"
    streams = int(g.integers(1, 5))
    widths = None
    if kind in ("multi", "multi_ids"):
        unit = 256 if dt == "bf16" else 64
        widths = [unit * int(g.integers(1, 4)) for _ in range(int(g.integers(2, 4)))]
    fmt = ("mxfp4" if (seed // 5) % 2 else "mxfp8") if kind == "mxfp8" else "bf16"
    if kind != "mxfp8" and seed % 7 == 3:
        layout = "both"          # the base held in both layouts (chosen by seed: other draws unchanged)
    return dict(kind=kind, dt=dt, ranks=ranks, tokens=tokens, d_in=d_in, d_out=d_out, layout=layout,
                streams=streams, widths=widths, seed=seed, fmt=fmt)


def _layer(plan, W0dev, A, B, scales, dt):
    from adapter_lora_segments_amd import PackedLoRALinear
    return PackedLoRALinear(plan, W0dev, [to_dev(a, dt) for a in A], [to_dev(b, dt) for b in B], scales)


def _z_pairs(plan, layer, off, P, n):
    zoff, rpad = plan.export("zoff"), plan.export("rpad")
    Zd = to_host_f64(layer.Z)
    out = []
    for v in range(n * P):
        i = v // P
        n_i = int(off[i + 1] - off[i])
        out.append(Zd[zoff[v]:zoff[v] + n_i * rpad[v]].reshape(n_i, rpad[v]))
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(N_CASES))
def test_sweep(seed):
    import torch
    from adapter_lora_segments_amd import Plan
    c = draw_case(seed)
    say(f"case sweep {seed}: {c}")
    dt, layout, kind = c["dt"], c["layout"], c["kind"]
    errs = {}
    zs_check = []
    if kind in ("multi", "multi_ids"):
        widths = c["widths"]
        P = len(widths)
        rk = [[c["ranks"][i]] * P if i % 2 == 0 else [max(1, c["ranks"][i] // (q + 1)) for q in range(P)]
              for i in range(len(c["ranks"]))]
        h = host_multi(seed, c["d_in"], widths, rk, c["tokens"], dt)
        Xh, dYh, order = h["X"], h["dY"], None
        if kind == "multi_ids":
            T = Xh.shape[0]
            order = np.random.default_rng(seed).permutation(T)
            ids = np.repeat(np.arange(len(rk)), np.diff(h["offsets"]))[order]
            Xh, dYh = np.ascontiguousarray(Xh[order]), np.ascontiguousarray(dYh[order])
            plan = Plan.multi_from_ids(ids, rk, c["d_in"], widths, dt, n_streams=c["streams"], w0_layout=layout)
        else:
            plan = Plan.multi(h["offsets"], rk, c["d_in"], widths, dt, n_streams=c["streams"], w0_layout=layout)
        W0h = h["W0"] if layout != "nk" else np.ascontiguousarray(h["W0"].T)
        flat = lambda x: [v for row in x for v in row]
        layer = _layer(plan, to_dev(W0h, dt), flat(h["A"]), flat(h["B"]), flat(h["scales"]), dt)
        X, dY = to_dev(Xh, dt), to_dev(dYh, dt)
        Y = layer.forward(X)
        dX = layer.backward(dY, X)
        torch.cuda.synchronize()
        # The oracle on the plan's grouped rows (grouped row g is the caller's
        # row perm[g]); its Y and dX go back to the caller's rows.
        perm = plan.export("perm") if order is not None else np.arange(Xh.shape[0])
        Xg, dYg = np.ascontiguousarray(Xh[perm]), np.ascontiguousarray(dYh[perm])
        Yg, Zo = om.forward_multi(Xg, h["W0"], h["A"], h["B"], h["scales"], h["offsets"], widths, dt)
        dXg, dAo, dBo, _ = om.backward_multi(dYg, Xg, h["W0"], h["A"], h["B"], h["scales"], h["offsets"],
                                             widths, dt)
        Yo, dXo = np.empty_like(Yg), np.empty_like(dXg)
        Yo[perm], dXo[perm] = Yg, dXg
        errs["Y"], errs["dX"] = ol.max_rel_err(to_host_f64(Y), Yo), ol.max_rel_err(to_host_f64(dX), dXo)
        zs = _z_pairs(plan, layer, h["offsets"], P, len(rk))
        for i in range(len(rk)):
            for q in range(P):
                v = i * P + q
                errs[f"dA{v}"] = ol.max_rel_err(to_host_f64(layer.dA[v]), dAo[i][q])
                errs[f"dB{v}"] = ol.max_rel_err(to_host_f64(layer.dB[v]), dBo[i][q])
                zs_check.append((f"Z{v}", zs[v], h["scales"][i][q] * Zo[i][q], rk[i][q]))
    else:
        w = custom_workload(f"sweep{seed}", dt, c["d_in"], c["d_out"], c["ranks"], c["tokens"], seed=seed,
                            n_streams=c["streams"])
        h = host_tensors(w, 0)
        off, n = h["offsets"], len(c["ranks"])
        X, dY, ids, W0o = h["X"], h["dY"], None, h["W0"]
        if kind == "ids":
            T = X.shape[0]
            order = np.random.default_rng(seed).permutation(T)
            ids = np.repeat(np.arange(n), np.diff(off))[order]
            X, dY = np.ascontiguousarray(X[order]), np.ascontiguousarray(dY[order])
            plan = Plan.from_ids(ids, h["ranks"], c["d_in"], c["d_out"], dt, n_streams=c["streams"],
                                 w0_layout=layout)
        else:
            plan = Plan(off, h["ranks"], c["d_in"], c["d_out"], dt, n_streams=c["streams"], w0_layout=layout,
                        w0_format=c["fmt"])
        if kind == "mxfp8":
            quant = quantize_mx4 if c["fmt"] == "mxfp4" else quantize_mx
            codes, sc = quant(ol.as_f64(h["W0"], "bf16"), layout)
            W0o = omx.dequant_w0(codes, sc, c["d_in"], c["d_out"], layout, fmt=c["fmt"])
            W0dev = torch.from_numpy(pack(codes, sc)).cuda()
        else:
            W0dev = to_dev(h["W0"] if layout != "nk" else np.ascontiguousarray(h["W0"].T), dt)
        layer = _layer(plan, W0dev, h["A"], h["B"], h["scales"], dt)
        Xd, dYd = to_dev(X, dt), to_dev(dY, dt)
        Y = layer.forward(Xd)
        dX = layer.backward(dYd, Xd)
        torch.cuda.synchronize()
        if kind == "ids":
            Yo, Zo = ol.forward_ids(X, W0o, h["A"], h["B"], h["scales"], ids, dt)
            dXo, dAo, dBo, _ = ol.backward_ids(dY, X, W0o, h["A"], h["B"], h["scales"], ids, dt)
        else:
            Yo, Zo = ol.forward(X, W0o, h["A"], h["B"], h["scales"], off, dt)
            dXo, dAo, dBo, _ = ol.backward(dY, X, W0o, h["A"], h["B"], h["scales"], off, dt)
        errs["Y"], errs["dX"] = ol.max_rel_err(to_host_f64(Y), Yo), ol.max_rel_err(to_host_f64(dX), dXo)
        zs = _z_pairs(plan, layer, plan.export("offsets"), 1, n)
        for i in range(n):
            errs[f"dA{i}"] = ol.max_rel_err(to_host_f64(layer.dA[i]), dAo[i])
            errs[f"dB{i}"] = ol.max_rel_err(to_host_f64(layer.dB[i]), dBo[i])
            zs_check.append((f"Z{i}", zs[i], float(h["scales"][i]) * Zo[i], int(h["ranks"][i])))
    for name, z, want, r in zs_check:
        errs[name] = ol.max_rel_err(z[:, :r], want)
        assert np.all(z[:, r:] == 0.0), f"{name}: padding columns not zero"
    worst = max(errs.items(), key=lambda kv: kv[1])
    say(f"  ksplit {plan.export('ksplit').tolist()}; worst {worst[0]} = {worst[1]:.3e} (tol {TOL[dt]:.0e})")
    bad = {k: v for k, v in errs.items() if not v <= TOL[dt]}
    assert not bad, bad
