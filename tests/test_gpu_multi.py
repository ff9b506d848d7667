"""Layers whose projections share one input (mlora_plan_multi) on the GPU.

- Against the oracle (oracle/multi.py) on small layers: Y, dX, every pair's
  saved activation Z' (padding columns exactly zero), dA and dB; bf16 with
  both W0 layouts and one to three stream groups, fp32 with both layouts;
  ranks 1..256, an adapter with no rows, projections of different widths;
  adapters whose padded ranks over the projections sum to at most 256
  (their shrink runs once for all projections), exactly 256, and above.
- The fused layer against one single-projection layer per projection over
  the same adapters: Y, Z', dA and dB are bit-identical (the same kernels
  visit the same extension steps, nano-batches and chunks in the same
  order); dX, a sum over projections, agrees within the bar.
- Full size, in the bench's launch configuration: the q/k/v and gate/up
  groups of the Llama-3-8B-shaped layer (16 adapters, 34816 rows): every
  pair's dA, dB and dZ element by element, and Y, dX and Z' on each
  adapter's first and last row plus 32 seeded rows inside it."""
import numpy as np
import pytest

from oracle import lora as ol
from oracle import multi as om
from tests.gpu_harness import TOL, say, to_dev, to_host_f64, workspace_dz
from tests.test_gpu_fullsize import stratified_rows
from workloads.multi import host_multi

CASES = [
    ("bf16", 256, [512, 256, 256], [[8, 8, 8], [64, 16, 33], [128, 1, 4], [256, 64, 32]], [150, 300, 0, 77], 1, "kn"),
    ("bf16", 320, [256, 512], [[16, 200], [3, 64], [256, 256]], [500, 9, 260], 3, "nk"),
    ("bf16", 256, [768, 768], [[256, 256], [32, 32]], [600, 333], 2, "kn"),
    # shrink over an adapter's projections at once: one adapter over the limit, one exactly at 256, and the
    # last one (padded ranks 3 x 32) in a 128-wide rank tile whose rows past the sum lie past A_cat^T
    ("bf16", 256, [256, 256, 512], [[256, 8, 8], [128, 64, 64], [1, 1, 1]], [200, 90, 131], 1, "nk"),
    ("fp32", 128, [128, 64, 64], [[4, 8, 2], [16, 1, 3]], [40, 57], 1, "kn"),
    ("fp32", 128, [64, 192], [[5, 7], [2, 2], [1, 33]], [13, 0, 29], 2, "nk"),
]


def _flat(nested):
    return [x for row in nested for x in row]


def _run(h, dt, layout, streams):
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    plan = Plan.multi(h["offsets"], h["ranks"], h["d_in"], h["widths"], dt, n_streams=streams,
                      w0_layout=layout)
    W0h = h["W0"] if layout == "kn" else np.ascontiguousarray(h["W0"].T)
    layer = PackedLoRALinear(plan, to_dev(W0h, dt), [to_dev(a, dt) for a in _flat(h["A"])],
                             [to_dev(b, dt) for b in _flat(h["B"])], _flat(h["scales"]))
    X, dY = to_dev(h["X"], dt), to_dev(h["dY"], dt)
    Y = layer.forward(X)
    dX = layer.backward(dY, X)
    torch.cuda.synchronize()
    return plan, layer, Y, dX


def _pair_z(plan, layer, off, v, i):
    zoff, rpad = plan.export("zoff"), plan.export("rpad")
    n_i = int(off[i + 1] - off[i])
    Zd = to_host_f64(layer.Z)
    return Zd[zoff[v]:zoff[v] + n_i * rpad[v]].reshape(n_i, rpad[v])


@pytest.mark.gpu
@pytest.mark.parametrize("dt,d_in,widths,ranks,tokens,streams,layout", CASES)
def test_multi_against_oracle(dt, d_in, widths, ranks, tokens, streams, layout):
    say(f"case multi {dt} d_in={d_in} widths={widths} ranks={ranks} tokens={tokens} streams={streams} {layout}")
    h = host_multi(11, d_in, widths, ranks, tokens, dt)
    plan, layer, Y, dX = _run(h, dt, layout, streams)
    Yo, Zo = om.forward_multi(h["X"], h["W0"], h["A"], h["B"], h["scales"], h["offsets"], widths, dt)
    dXo, dAo, dBo, _ = om.backward_multi(h["dY"], h["X"], h["W0"], h["A"], h["B"], h["scales"], h["offsets"],
                                         widths, dt)
    errs = {"Y": ol.max_rel_err(to_host_f64(Y), Yo), "dX": ol.max_rel_err(to_host_f64(dX), dXo)}
    P = len(widths)
    off = h["offsets"]
    for i in range(len(tokens)):
        for q in range(P):
            v = i * P + q
            r = ranks[i][q]
            errs[f"dA{i},{q}"] = ol.max_rel_err(to_host_f64(layer.dA[v]), dAo[i][q])
            errs[f"dB{i},{q}"] = ol.max_rel_err(to_host_f64(layer.dB[v]), dBo[i][q])
            z = _pair_z(plan, layer, off, v, i)
            errs[f"Z{i},{q}"] = ol.max_rel_err(z[:, :r], h["scales"][i][q] * Zo[i][q])
            assert np.all(z[:, r:] == 0.0), f"padded Z' columns of pair {i},{q} not zero"
    worst = max(errs.items(), key=lambda kv: kv[1])
    say(f"  worst {worst[0]} = {worst[1]:.3e} (tol {TOL[dt]:.0e})")
    bad = {k: e for k, e in errs.items() if not e <= TOL[dt]}
    assert not bad, bad


@pytest.mark.gpu
@pytest.mark.parametrize("dt,d_in,widths,ranks,tokens,streams,layout",
                         [CASES[0], CASES[1], CASES[3], CASES[4]])
def test_multi_equals_separate_layers(dt, d_in, widths, ranks, tokens, streams, layout):
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    say(f"case fused vs separate {dt} widths={widths} streams={streams} {layout}")
    h = host_multi(12, d_in, widths, ranks, tokens, dt)
    plan, layer, Y, dX = _run(h, dt, layout, streams)
    Yf, dXf = to_host_f64(Y), to_host_f64(dX)
    P = len(widths)
    cols = om.columns(widths)
    off = h["offsets"]
    dX_sum = np.zeros_like(dXf)
    for q in range(P):
        Wq = np.ascontiguousarray(h["W0"][:, cols[q]:cols[q + 1]])
        rq = [ranks[i][q] for i in range(len(tokens))]
        pl = Plan(off, rq, d_in, widths[q], dt, n_streams=streams, w0_layout=layout)
        lay = PackedLoRALinear(pl, to_dev(Wq if layout == "kn" else np.ascontiguousarray(Wq.T), dt),
                               [to_dev(h["A"][i][q], dt) for i in range(len(tokens))],
                               [to_dev(h["B"][i][q], dt) for i in range(len(tokens))],
                               [h["scales"][i][q] for i in range(len(tokens))])
        X = to_dev(h["X"], dt)
        Yq = lay.forward(X)
        dXq = lay.backward(to_dev(np.ascontiguousarray(h["dY"][:, cols[q]:cols[q + 1]]), dt), X)
        torch.cuda.synchronize()
        assert np.array_equal(Yf[:, cols[q]:cols[q + 1]], to_host_f64(Yq)), f"Y of projection {q} differs"
        dX_sum += to_host_f64(dXq)
        for i in range(len(tokens)):
            v = i * P + q
            assert np.array_equal(to_host_f64(layer.dA[v]), to_host_f64(lay.dA[i])), f"dA {i},{q}"
            assert np.array_equal(to_host_f64(layer.dB[v]), to_host_f64(lay.dB[i])), f"dB {i},{q}"
            assert np.array_equal(_pair_z(plan, layer, off, v, i), _pair_z(pl, lay, off, i, i)), f"Z {i},{q}"
    e = ol.max_rel_err(dXf, dX_sum)
    say(f"  Y, Z', dA, dB bit-identical; dX vs sum of separate dX: {e:.3e}")
    assert e <= TOL[dt]


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.gpu
@pytest.mark.parametrize("group", ["qkv", "gate_up"])
def test_multi_full_size_llama3(group):
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    from workloads import load_workload
    from workloads.multi import LAYER_GROUPS, device_multi
    w = load_workload("llama3_8b_layer", 0)
    projs = dict(LAYER_GROUPS[w.name])[group]
    d = device_multi(w, projs)
    widths = d["widths"]
    say(f"case full-size {w.name} {group}: d_in {d['d_in']}, widths {widths}, T={w.T}, {w.n} adapters")
    plan = Plan.multi(d["offsets"], d["ranks"], d["d_in"], widths, "bf16", n_streams=w.n_streams)
    layer = PackedLoRALinear(plan, d["W0"], _flat(d["A"]), _flat(d["B"]), _flat(d["scales"]))
    X, dY = d["X"][0], d["dY"][0]
    Y = layer.forward(X)
    dX = layer.backward(dY, X)
    torch.cuda.synchronize()
    off = d["offsets"]
    Xh, dYh, W0h = _bits(X), _bits(dY), _bits(d["W0"])
    Ah = [[_bits(a) for a in row] for row in d["A"]]
    Bh = [[_bits(b) for b in row] for row in d["B"]]
    rng = np.random.default_rng(23)
    rows = stratified_rows(off, rng)
    rt = torch.from_numpy(rows).cuda()
    gY = Y.index_select(0, rt).float().cpu().numpy()
    gdX = dX.index_select(0, rt).float().cpu().numpy()
    Zd = layer.Z.float().cpu().numpy()
    dZd = workspace_dz(plan, layer)
    gA = [t.double().cpu().numpy() for t in layer.dA]
    gB = [t.double().cpu().numpy() for t in layer.dB]
    say(f"  GPU done; oracle on {len(rows)} rows and the full weight gradients")
    Ys, dXs, Zs = om.sampled_rows_multi(rows, Xh, W0h, Ah, Bh, d["scales"], off, widths, dY=dYh, dtype="bf16")
    errs = {"Y": ol.max_rel_err(gY, Ys), "dX": ol.max_rel_err(gdX, dXs)}
    P = len(widths)
    zoff, rpad = plan.export("zoff"), plan.export("rpad")
    own = np.searchsorted(off, rows, side="right") - 1
    gz, wz = [], []
    for k, (t, i) in enumerate(zip(rows, own)):
        for q in range(P):
            v = i * P + q
            gz.append(Zd[zoff[v] + (t - off[i]) * rpad[v]:][:d["ranks"][i][q]])
            wz.append(Zs[k][q])
    errs["Z"] = ol.max_rel_err(np.concatenate(gz), np.concatenate(wz))
    _, dA, dB, dZ = om.backward_multi(dYh, Xh, W0h, Ah, Bh, d["scales"], off, widths, "bf16", want_dx=False)
    for i in range(w.n):
        n_i = int(off[i + 1] - off[i])
        for q in range(P):
            v, r = i * P + q, int(d["ranks"][i][q])
            errs[f"dA{i},{q}"] = ol.max_rel_err(gA[v], dA[i][q])
            errs[f"dB{i},{q}"] = ol.max_rel_err(gB[v], dB[i][q])
            dzv = dZd[zoff[v]:zoff[v] + n_i * rpad[v]].reshape(n_i, rpad[v])
            errs[f"dZ{i},{q}"] = ol.max_rel_err(dzv[:, :r], dZ[i][q])
            assert np.all(dzv[:, r:] == 0.0), f"padded dZ columns of pair {v} not zero"
    worst = max(errs.items(), key=lambda kv: kv[1])
    say(f"  {group}: {len(rows)} rows, every dA/dB/dZ element, worst {worst[0]} = {worst[1]:.3e}")
    bad = {k: e for k, e in errs.items() if not e <= TOL["bf16"]}
    assert not bad, bad
