"""Full-size parity of the larger workloads (Llama-3-8B layer, 64 Zipf-sized
adapters, 70B MLP pair on four streams), in the launch configuration bench.py
uses: default plan options and the workload's stream count.

What is compared with the float64 oracle (PLoRA: Efficient Concurrent LoRA
Training for Large Language Models, §9.2, Cases 1-3, and §2.1):
- every dA_i and dB_i, element by element, and the backward's intermediate
  dZ_i = s_i dY_i B_i^T on every row (the oracle's streamed backward without
  dX: about 4 sum_i n_i r_i (d_in + d_out) flops);
- Y, dX and the saved activation Z' on every adapter's first and last row
  plus 32 seeded rows inside it (all rows of smaller adapters), row by row
  (a full float64 dX or Y would be 2 T d_in d_out flops per tensor).
Inputs are drawn on the device; the oracle reads the same bf16 bits copied
back to the host."""
import numpy as np
import pytest

from tests.gpu_harness import TOL, say, workspace_dz
from oracle import lora as ol
from workloads import load_workload
from workloads.tensors import device_tensors

CASES = ([("llama3_8b_layer", p) for p in range(7)] + [("nano_stress", 0)] +
         [("mlp70b_pair", 0), ("mlp70b_pair", 1)])
ROWS_PER_ADAPTER = 32


def stratified_rows(offsets, rng, per=ROWS_PER_ADAPTER):
    """Each non-empty segment's first and last row plus ``per`` distinct
    seeded rows inside it (every row when it has fewer)."""
    rows = []
    o = [int(v) for v in offsets]
    for i in range(len(o) - 1):
        lo, hi = o[i], o[i + 1]
        if hi > lo:
            rows += [lo, hi - 1]
            rows += rng.choice(np.arange(lo, hi), size=min(per, hi - lo), replace=False).tolist()
    return np.unique(np.asarray(rows, dtype=np.int64))


def _bits(t):
    """bf16 device tensor -> host uint16 bit patterns."""
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.gpu
@pytest.mark.parametrize("name,proj", CASES)
def test_full_size(name, proj):
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
    rng = np.random.default_rng(17 + proj)
    rows = stratified_rows(off, rng)
    rows_t = torch.from_numpy(rows).cuda()
    gY = Y.index_select(0, rows_t).float().cpu().numpy()
    gdX = dX.index_select(0, rows_t).float().cpu().numpy()
    Zd = layer.Z.float().cpu().numpy()
    dZd = workspace_dz(plan, layer)
    gA = [t.double().cpu().numpy() for t in layer.dA]
    gB = [t.double().cpu().numpy() for t in layer.dB]
    Xh, dYh, W0h = _bits(X), _bits(dY), _bits(d["W0"])
    Ah = [_bits(a) for a in d["A"]]
    Bh = [_bits(b) for b in d["B"]]
    del Y, dX, layer, d
    torch.cuda.empty_cache()
    say(f"  GPU done; oracle on {len(rows)} rows and the full weight gradients")

    Ys, dXs, Zs = ol.sampled_rows(rows, Xh, W0h, Ah, Bh, sc, off, dY=dYh, dtype="bf16", with_z=True)
    errs = {"Y": ol.max_rel_err(gY, Ys), "dX": ol.max_rel_err(gdX, dXs)}
    zoff, rpad = plan.export("zoff"), plan.export("rpad")
    own = ol.adapter_of_rows(off, rows)
    gz = np.concatenate([Zd[zoff[i] + (t - off[i]) * rpad[i]:][:int(w.ranks[i])] for t, i in zip(rows, own)])
    errs["Z"] = ol.max_rel_err(gz, np.concatenate(Zs))

    _, dA, dB, dZ = ol.backward(dYh, Xh, W0h, Ah, Bh, sc, off, "bf16", want_dx=False)
    for i in range(w.n):
        r, n_i = int(w.ranks[i]), int(off[i + 1] - off[i])
        errs[f"dA{i}"] = ol.max_rel_err(gA[i], dA[i])
        errs[f"dB{i}"] = ol.max_rel_err(gB[i], dB[i])
        dzi = dZd[zoff[i]:zoff[i] + n_i * rpad[i]].reshape(n_i, rpad[i])
        errs[f"dZ{i}"] = ol.max_rel_err(dzi[:, :r], dZ[i])
        assert np.all(dzi[:, r:] == 0.0), f"padded dZ columns of adapter {i} not zero"
    worst = max(errs.items(), key=lambda kv: kv[1])
    say(f"  {name}/{p.name}: {len(rows)} rows, every dA/dB/dZ element, worst {worst[0]} = {worst[1]:.3e}")
    bad = {k: v for k, v in errs.items() if not v <= TOL["bf16"]}
    assert not bad, f"{name}/{p.name}: tolerance {TOL['bf16']} exceeded: {bad}"
