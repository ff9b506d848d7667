"""Helpers for the GPU parity tests: run the HIP path through the C interface
on seeded inputs and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

from oracle import lora as ol
from workloads.configs import Workload, Projection
from workloads.tensors import host_tensors

TOL = {"bf16": 2e-2, "fp32": 1e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def to_host_f64(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def custom_workload(name, dtype, d_in, d_out, ranks, tokens, scales=None, seed=0, n_streams=1):
    w = Workload(name, dtype, [Projection("p", d_in, d_out)], list(ranks), list(tokens),
                 n_streams=n_streams, seed=seed)
    if scales is not None:
        w.scales = list(scales)
    return w


def run_gpu(w: Workload, proj=0, w0_layout="kn", n_streams=None, nano_rows=0, h=None,
            want_dx=True, chunk_min=0, chunk_max=0, chunk_per_rank=0, wg_overlap="auto"):
    """Run forward+backward on the GPU.  Returns (host inputs, outputs dict)."""
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    if h is None:
        h = host_tensors(w, proj)
    dt = w.dtype
    plan = Plan(h["offsets"], h["ranks"], h["d_in"], h["d_out"], dt,
                n_streams=n_streams if n_streams is not None else w.n_streams,
                nano_rows=nano_rows, w0_layout=w0_layout, chunk_min=chunk_min,
                chunk_max=chunk_max, chunk_per_rank=chunk_per_rank, wg_overlap=wg_overlap)
    W0h = h["W0"] if w0_layout == "kn" else np.ascontiguousarray(h["W0"].T)
    W0 = to_dev(W0h, dt)
    A = [to_dev(a, dt) for a in h["A"]]
    B = [to_dev(b, dt) for b in h["B"]]
    layer = PackedLoRALinear(plan, W0, A, B, h["scales"])
    X = to_dev(h["X"], dt)
    dY = to_dev(h["dY"], dt)
    Y = layer.forward(X)
    dX = layer.backward(dY, X, want_dx=want_dx)
    torch.cuda.synchronize()
    out = {
        "dZ": workspace_dz(plan, layer),
        "Y": to_host_f64(Y),
        "dX": to_host_f64(dX) if want_dx else None,
        "dA": [to_host_f64(t) for t in layer.dA],
        "dB": [to_host_f64(t) for t in layer.dB],
        "Z": to_host_f64(layer.Z),
        "plan": plan,
        "layer": layer,
        "dev": dict(X=X, dY=dY, Y=Y, dX=dX),
    }
    return h, out


def workspace_dz(plan, layer):
    """dZ = s dY B^T as the last backward left it in the workspace (layout of
    Z'), float64 on the host."""
    import torch
    i = plan.info
    esz = 2 if plan.dtype == "bf16" else 4
    raw = layer.ws[i["dz_offset"]:i["dz_offset"] + i["z_elems"] * esz]
    t = raw.view(torch.bfloat16 if esz == 2 else torch.float32)
    return to_host_f64(t)


def compare(w: Workload, h, out, tol=None, what=""):
    """Full comparison against the oracle (small and medium sizes)."""
    dt = w.dtype
    tol = TOL[dt] if tol is None else tol
    Y, Zs = ol.forward(h["X"], h["W0"], h["A"], h["B"], h["scales"], h["offsets"], dt)
    dX, dA, dB, dZ = ol.backward(h["dY"], h["X"], h["W0"], h["A"], h["B"], h["scales"],
                                 h["offsets"], dt, want_dx=out["dX"] is not None)
    errs = {"Y": ol.max_rel_err(out["Y"], Y)}
    if out["dX"] is not None:
        errs["dX"] = ol.max_rel_err(out["dX"], dX)
    plan = out["plan"]
    zoff = plan.export("zoff")
    rpad = plan.export("rpad")
    o = h["offsets"]
    for i in range(len(h["ranks"])):
        r = int(h["ranks"][i])
        errs[f"dA{i}"] = ol.max_rel_err(out["dA"][i], dA[i])
        errs[f"dB{i}"] = ol.max_rel_err(out["dB"][i], dB[i])
        n_i = int(o[i + 1] - o[i])
        zi = out["Z"][zoff[i]:zoff[i] + n_i * rpad[i]].reshape(n_i, rpad[i])
        errs[f"Z{i}"] = ol.max_rel_err(zi[:, :r], float(h["scales"][i]) * Zs[i])
        assert np.all(zi[:, r:] == 0.0), f"{what}: padded Z columns of adapter {i} not zero"
        # the backward's intermediate dZ_i = s_i dY_i B_i^T (PLoRA §9.2, Case 2)
        dzi = out["dZ"][zoff[i]:zoff[i] + n_i * rpad[i]].reshape(n_i, rpad[i])
        errs[f"dZ{i}"] = ol.max_rel_err(dzi[:, :r], dZ[i])
        assert np.all(dzi[:, r:] == 0.0), f"{what}: padded dZ columns of adapter {i} not zero"
    bad = {k: v for k, v in errs.items() if not (v <= tol)}
    worst = max(errs.items(), key=lambda kv: kv[1])
    say(f"  {what}: worst {worst[0]} = {worst[1]:.3e} (tol {tol:.0e})")
    assert not bad, f"{what}: tolerance {tol} exceeded: {bad}"
    return errs
