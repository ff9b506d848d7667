"""GEMM launches with few output tiles split K across workgroups (rule 9 of
the plan): the parts' fp32 tiles are added in part order by a second
kernel.  These cases put every split path on the GPU against the oracle:
forward and dX splits of different factors, the last part's extension steps,
parts with an odd number of 32-deep sub-steps,
rows in the caller's order (ids), several stream groups each with its own
partial region, several projections sharing the input, and both W0 layouts;
two runs must be bitwise identical."""
import numpy as np
import pytest

from oracle import lora as ol
from tests.gpu_harness import TOL, compare, custom_workload, run_gpu, say, to_dev, to_host_f64

SEG_CASES = [
    # name, d_in, d_out, ranks, tokens, streams, layout, expected ksplit per group
    ("one adapter 512x2048^2", 2048, 2048, [16], [512], 1, "kn", [[8, 8]]),
    ("tall dX split", 512, 8192, [8, 64], [120, 180], 1, "nk", [[2, 16]]),
    ("three groups", 1024, 1536, [4, 32, 256, 16, 8], [100, 40, 300, 0, 77], 3, "kn", None),
    ("ragged, ranks 1-256", 768, 1024, [1, 33, 256, 100], [17, 250, 33, 64], 1, "nk", None),
    # 34 sub-steps of 32 split 9+9+9+7: every part has a 64-deep step with one
    # half past its main K (zero page, or the first extension sub-step in the
    # last part); N = 1088 leaves a ragged column tile
    ("odd sub-steps per part", 1088, 1088, [16, 48, 5], [150, 250, 90], 1, "kn", [[4, 4]]),
    ("odd sub-steps per part, nk", 1088, 1088, [16, 48, 5], [150, 250, 90], 1, "nk", [[4, 4]]),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,d_in,d_out,ranks,tokens,streams,layout,ks", SEG_CASES)
def test_split_k_against_oracle(name, d_in, d_out, ranks, tokens, streams, layout, ks):
    w = custom_workload(name, "bf16", d_in, d_out, ranks, tokens, seed=5, n_streams=streams)
    say(f"case split-k {name}: {d_in}x{d_out}, ranks {ranks}, tokens {tokens}, {streams} stream(s), {layout}")
    h, out = run_gpu(w, w0_layout=layout)
    got = out["plan"].export("ksplit").tolist()
    say(f"  ksplit per group (forward, dX): {got}")
    if ks is not None:
        assert got == ks
    assert any(s > 1 for row in got for s in row), "case does not split"
    compare(w, h, out, what=name)


@pytest.mark.gpu
def test_split_k_bitwise_repeatable():
    import torch
    w = custom_workload("repeat", "bf16", 2048, 2048, [16, 64], [300, 212], seed=6)
    say("case split-k repeatability")
    h, out = run_gpu(w)
    layer, d = out["layer"], out["dev"]
    Y2 = layer.forward(d["X"])
    dX2 = layer.backward(d["dY"], d["X"])
    torch.cuda.synchronize()
    assert np.array_equal(to_host_f64(Y2), out["Y"]) and np.array_equal(to_host_f64(dX2), out["dX"])


@pytest.mark.gpu
def test_split_k_with_ids_and_projections():
    """Split-K under a row permutation (plan from ids) and under several
    projections sharing the input."""
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    from oracle import multi as om
    from workloads.multi import host_multi
    from workloads.tensors import host_tensors
    say("case split-k with shuffled ids")
    w = custom_workload("ids", "bf16", 1024, 2048, [8, 128, 32], [150, 260, 90], seed=7)
    h = host_tensors(w, 0)
    T = h["X"].shape[0]
    grouped = np.repeat(np.arange(3), np.diff(h["offsets"]))
    order = np.random.default_rng(3).permutation(T)
    ids = grouped[order]
    X, dY = np.ascontiguousarray(h["X"][order]), np.ascontiguousarray(h["dY"][order])
    plan = Plan.from_ids(ids, h["ranks"], 1024, 2048, "bf16")
    assert any(s > 1 for row in plan.export("ksplit").tolist() for s in row)
    layer = PackedLoRALinear(plan, to_dev(h["W0"], "bf16"), [to_dev(a, "bf16") for a in h["A"]],
                             [to_dev(b, "bf16") for b in h["B"]], h["scales"])
    Xd, dYd = to_dev(X, "bf16"), to_dev(dY, "bf16")
    Y = layer.forward(Xd)
    dX = layer.backward(dYd, Xd)
    torch.cuda.synchronize()
    Yo, _ = ol.forward_ids(X, h["W0"], h["A"], h["B"], h["scales"], ids, "bf16")
    dXo, dAo, dBo, _ = ol.backward_ids(dY, X, h["W0"], h["A"], h["B"], h["scales"], ids, "bf16")
    errs = {"Y": ol.max_rel_err(to_host_f64(Y), Yo), "dX": ol.max_rel_err(to_host_f64(dX), dXo)}
    for i in range(3):
        errs[f"dA{i}"] = ol.max_rel_err(to_host_f64(layer.dA[i]), dAo[i])
        errs[f"dB{i}"] = ol.max_rel_err(to_host_f64(layer.dB[i]), dBo[i])
    say(f"  ids: worst {max(errs.items(), key=lambda kv: kv[1])}")
    assert all(e <= TOL["bf16"] for e in errs.values()), errs

    say("case split-k with projections sharing the input")
    widths = [1024, 512, 512]
    ranks = [[8, 8, 8], [64, 16, 128]]
    hm = host_multi(8, 1024, widths, ranks, [200, 111], "bf16")
    plan = Plan.multi(hm["offsets"], ranks, 1024, widths, "bf16", w0_layout="nk")
    assert any(s > 1 for row in plan.export("ksplit").tolist() for s in row)
    flat = lambda nested: [x for row in nested for x in row]
    layer = PackedLoRALinear(plan, to_dev(np.ascontiguousarray(hm["W0"].T), "bf16"),
                             [to_dev(a, "bf16") for a in flat(hm["A"])], [to_dev(b, "bf16") for b in flat(hm["B"])],
                             flat(hm["scales"]))
    Xd, dYd = to_dev(hm["X"], "bf16"), to_dev(hm["dY"], "bf16")
    Y = layer.forward(Xd)
    dX = layer.backward(dYd, Xd)
    torch.cuda.synchronize()
    Yo, _ = om.forward_multi(hm["X"], hm["W0"], hm["A"], hm["B"], hm["scales"], hm["offsets"], widths, "bf16")
    dXo, dAo, dBo, _ = om.backward_multi(hm["dY"], hm["X"], hm["W0"], hm["A"], hm["B"], hm["scales"],
                                         hm["offsets"], widths, "bf16")
    errs = {"Y": ol.max_rel_err(to_host_f64(Y), Yo), "dX": ol.max_rel_err(to_host_f64(dX), dXo)}
    for i in range(2):
        for q in range(3):
            errs[f"dA{i},{q}"] = ol.max_rel_err(to_host_f64(layer.dA[3 * i + q]), dAo[i][q])
            errs[f"dB{i},{q}"] = ol.max_rel_err(to_host_f64(layer.dB[3 * i + q]), dBo[i][q])
    say(f"  projections: worst {max(errs.items(), key=lambda kv: kv[1])}")
    assert all(e <= TOL["bf16"] for e in errs.values()), errs
