"""Plans from per-token adapter ids (mlora_plan_from_ids) on the GPU.

Rows arrive in the caller's order with shuffled adapter ids: Y, dX, dA, dB
and Z' are compared with the oracle's forward_ids / backward_ids, on the
bf16 path (both W0 layouts, one and three stream groups, an adapter with no
rows) and the fp32 path.  Ids already in adapter order must give bitwise
the results of the segment plan (same kernels, identity permutation)."""
import numpy as np
import pytest

from oracle import lora as ol
from tests.gpu_harness import TOL, custom_workload, say, to_dev, to_host_f64
from workloads.tensors import host_tensors


def _case(w, seed, shuffle=True):
    h = host_tensors(w, 0)
    T = h["X"].shape[0]
    grouped_ids = np.repeat(np.arange(len(h["ranks"])), np.diff(h["offsets"]))
    order = np.random.default_rng(seed).permutation(T) if shuffle else np.arange(T)
    # caller row t is grouped row order[t]
    return h, np.ascontiguousarray(h["X"][order]), np.ascontiguousarray(h["dY"][order]), grouped_ids[order]


def _run(h, X, dY, plan, dt, w0_layout):
    import torch
    from adapter_lora_segments_amd import PackedLoRALinear
    W0h = h["W0"] if w0_layout == "kn" else np.ascontiguousarray(h["W0"].T)
    layer = PackedLoRALinear(plan, to_dev(W0h, dt), [to_dev(a, dt) for a in h["A"]],
                             [to_dev(b, dt) for b in h["B"]], h["scales"])
    Xd, dYd = to_dev(X, dt), to_dev(dY, dt)
    Y = layer.forward(Xd)
    dX = layer.backward(dYd, Xd)
    torch.cuda.synchronize()
    return {"Y": to_host_f64(Y), "dX": to_host_f64(dX), "dA": [to_host_f64(t) for t in layer.dA],
            "dB": [to_host_f64(t) for t in layer.dB], "Z": to_host_f64(layer.Z)}


CASES = [
    ("bf16", 256, 320, [8, 64, 200, 3], [150, 300, 77, 0], 1, "kn"),
    ("bf16", 256, 320, [8, 64, 200, 3], [150, 300, 77, 0], 3, "kn"),
    ("bf16", 320, 256, [16, 33, 1], [500, 9, 260], 1, "nk"),
    ("fp32", 128, 192, [4, 8, 2], [40, 0, 57], 1, "kn"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("dt,d_in,d_out,ranks,tokens,streams,layout", CASES)
def test_shuffled_ids_against_oracle(dt, d_in, d_out, ranks, tokens, streams, layout):
    from adapter_lora_segments_amd import Plan
    say(f"case ids {dt} {d_in}x{d_out} ranks {ranks} tokens {tokens} streams {streams} {layout}")
    w = custom_workload("ids", dt, d_in, d_out, ranks, tokens, seed=5)
    h, X, dY, ids = _case(w, seed=11)
    plan = Plan.from_ids(ids, h["ranks"], d_in, d_out, dt, n_streams=streams, w0_layout=layout)
    assert np.array_equal(plan.export("perm")[np.argsort(plan.export("perm"))], np.arange(len(ids)))
    got = _run(h, X, dY, plan, dt, layout)
    Y, Zs = ol.forward_ids(X, h["W0"], h["A"], h["B"], h["scales"], ids, dt)
    dX, dA, dB, _ = ol.backward_ids(dY, X, h["W0"], h["A"], h["B"], h["scales"], ids, dt)
    errs = {"Y": ol.max_rel_err(got["Y"], Y), "dX": ol.max_rel_err(got["dX"], dX)}
    zoff, rpad, off = plan.export("zoff"), plan.export("rpad"), plan.export("offsets")
    for i, r in enumerate(ranks):
        errs[f"dA{i}"] = ol.max_rel_err(got["dA"][i], dA[i])
        errs[f"dB{i}"] = ol.max_rel_err(got["dB"][i], dB[i])
        n_i = int(off[i + 1] - off[i])
        zi = got["Z"][zoff[i]:zoff[i] + n_i * rpad[i]].reshape(n_i, rpad[i])
        errs[f"Z{i}"] = ol.max_rel_err(zi[:, :r], float(h["scales"][i]) * Zs[i])
    worst = max(errs.items(), key=lambda kv: kv[1])
    say(f"  worst {worst[0]} = {worst[1]:.3e} (tol {TOL[dt]:.0e})")
    bad = {k: v for k, v in errs.items() if not v <= TOL[dt]}
    assert not bad, f"tolerance {TOL[dt]} exceeded: {bad}"


@pytest.mark.gpu
@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_grouped_ids_match_segment_plan_bitwise(dt):
    from adapter_lora_segments_amd import Plan
    say(f"case ids grouped vs segments {dt}")
    w = custom_workload("ids_grouped", dt, 256, 192, [8, 40, 130], [70, 260, 33], seed=6)
    h, X, dY, ids = _case(w, seed=0, shuffle=False)
    a = _run(h, X, dY, Plan.from_ids(ids, h["ranks"], 256, 192, dt), dt, "kn")
    b = _run(h, X, dY, Plan(h["offsets"], h["ranks"], 256, 192, dt), dt, "kn")
    for k in ("Y", "dX", "Z"):
        assert np.array_equal(a[k], b[k]), k
    for i in range(3):
        assert np.array_equal(a["dA"][i], b["dA"][i]) and np.array_equal(a["dB"][i], b["dB"][i]), i
