"""Full-size parity of the larger workloads (Llama-3-8B layer, 64 Zipf-sized
adapters, 70B MLP pair on four streams), in the launch configuration bench.py
uses: default plan options and the workload's stream count.

A full float64 oracle at these sizes takes minutes per projection, so:
- Y, dX and the saved activation Z' are checked exactly on sampled rows
  (every adapter's first and last row plus one inside), row by row;
- dA_i and dB_i are checked through random projections: dA_i u and dB_i v
  against the oracle's chains of matrix-vector products over all rows
  (Freivalds' check), which holds at any size.
Inputs are drawn on the device; the oracle reads the same bf16 bits copied
back to the host."""
import numpy as np
import pytest

from tests.gpu_harness import TOL, say
from oracle import lora as ol
from workloads import load_workload
from workloads.tensors import device_tensors

CASES = ([("llama3_8b_layer", p) for p in range(7)] + [("nano_stress", 0)] +
         [("mlp70b_pair", 0), ("mlp70b_pair", 1)])


def _sample_rows(offsets, rng):
    rows = []
    o = [int(v) for v in offsets]
    for i in range(len(o) - 1):
        if o[i + 1] > o[i]:
            rows += [o[i], o[i + 1] - 1, int(rng.integers(o[i], o[i + 1]))]
    return np.unique(np.asarray(rows, dtype=np.int64))


def _bits(t):
    """bf16 device tensor -> host uint16 bit patterns."""
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.gpu
@pytest.mark.parametrize("name,proj", CASES)
def test_full_size_sampled(name, proj):
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    w = load_workload(name, 0)
    p = w.projections[proj]
    say(f"case {name} projection {p.name} ({p.d_in}x{p.d_out}, T={w.T}, "
        f"{w.n} adapters, {w.n_streams} stream(s))")
    d = device_tensors(w, proj)
    plan = Plan(d["offsets"], d["ranks"], p.d_in, p.d_out, "bf16", n_streams=w.n_streams)
    layer = PackedLoRALinear(plan, d["W0"], d["A"], d["B"], d["scales"])
    X, dY = d["X"][0], d["dY"][0]
    Y = layer.forward(X)
    dX = layer.backward(dY, X)
    torch.cuda.synchronize()

    off, sc = d["offsets"], d["scales"]
    Xh, dYh, W0h = _bits(X), _bits(dY), _bits(d["W0"])
    Ah = [_bits(a) for a in d["A"]]
    Bh = [_bits(b) for b in d["B"]]
    rng = np.random.default_rng(17 + proj)
    rows = _sample_rows(off, rng)
    rows_t = torch.from_numpy(rows).cuda()
    gY = Y.index_select(0, rows_t).float().cpu().numpy()
    gdX = dX.index_select(0, rows_t).float().cpu().numpy()
    Ys, dXs, Zs = ol.sampled_rows(rows, Xh, W0h, Ah, Bh, sc, off, dY=dYh, dtype="bf16", with_z=True)
    errs = {"Y": ol.max_rel_err(gY, Ys), "dX": ol.max_rel_err(gdX, dXs)}

    # saved activation of the sampled rows, in the plan's layout
    zoff, rpad = plan.export("zoff"), plan.export("rpad")
    Zd = layer.Z.float().cpu().numpy()
    own = ol.adapter_of_rows(off, rows)
    gz = np.concatenate([Zd[zoff[i] + (t - off[i]) * rpad[i]:][:int(d["ranks"][i])] for t, i in zip(rows, own)])
    errs["Z"] = ol.max_rel_err(gz, np.concatenate(Zs))

    U = [rng.standard_normal(int(r)) for r in d["ranks"]]
    V = [rng.standard_normal(p.d_out) for _ in d["ranks"]]
    pa, pb = ol.projected_grads(Xh, dYh, Ah, Bh, sc, off, U, V, dtype="bf16", chunk=2048)
    for i in range(w.n):
        gA = layer.dA[i].double().cpu().numpy()
        gB = layer.dB[i].double().cpu().numpy()
        errs[f"dA{i}.u"] = ol.max_rel_err(gA @ U[i], pa[i])
        errs[f"dB{i}.v"] = ol.max_rel_err(gB @ V[i], pb[i])
    worst = max(errs.items(), key=lambda kv: kv[1])
    say(f"  {name}/{p.name}: {len(rows)} sampled rows, worst {worst[0]} = {worst[1]:.3e}")
    bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
    assert not bad, f"{name}/{p.name}: tolerance {TOL['bf16']} exceeded: {bad}"
