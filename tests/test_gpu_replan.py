"""Adapters join and leave between steps (the tLoRA page's elastic shared
super-model, one GPU): a pool of adapters keeps its device tensors, and each
step builds a new plan over the adapters active then, with new token
counts, ranks in another order, a different number of stream groups, and
rows given either as segments or as shuffled per-token ids.  Every step's
Y, dX, dA_i, dB_i, Z' and dZ are checked against the oracle, so nothing a
plan leaves in the layer's buffers carries into the next."""
from types import SimpleNamespace

import numpy as np
import pytest

from tests.gpu_harness import compare, say, to_dev, workspace_dz, to_host_f64
from workloads.tensors import f32_to_bf16_bits

D_IN, D_OUT = 512, 768
POOL_RANKS = [8, 64, 16, 200, 4, 33, 128]
# (active adapters in the layer's order, their token counts, stream groups, rows as ids)
STEPS = [
    ([0, 1, 2, 3], [300, 200, 0, 400], 1, False),
    ([4, 0, 5, 2], [100, 350, 50, 500], 2, False),      # 1 and 3 leave, 4 and 5 join
    ([6, 5, 4, 3, 2, 1, 0], [90, 0, 270, 33, 400, 128, 256], 3, True),
    ([2], [640], 1, False),
]


@pytest.mark.gpu
def test_adapters_join_and_leave_between_steps():
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    rng = np.random.default_rng(71)
    bits = lambda shape, std: f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32) * std)
    W0h = bits((D_IN, D_OUT), 0.02)
    Ah = [bits((D_IN, r), D_IN ** -0.5) for r in POOL_RANKS]
    Bh = [bits((r, D_OUT), 0.01) for r in POOL_RANKS]
    W0 = to_dev(W0h, "bf16")
    A = [to_dev(a, "bf16") for a in Ah]          # the pool's device tensors, kept across plans
    B = [to_dev(b, "bf16") for b in Bh]
    for k, (active, tokens, streams, ids) in enumerate(STEPS):
        say(f"case replan step {k}: adapters {active} tokens {tokens} streams {streams} ids {ids}")
        ranks = [POOL_RANKS[i] for i in active]
        scales = [16.0 / r for r in ranks]
        off = np.concatenate([[0], np.cumsum(tokens)]).astype(np.int64)
        T = int(off[-1])
        X, dY = bits((T, D_IN), 1.0), bits((T, D_OUT), 1.0)
        if ids:
            tok = np.repeat(np.arange(len(active)), tokens)
            perm = rng.permutation(T)
            plan = Plan.from_ids(tok[perm], ranks, D_IN, D_OUT, "bf16", n_streams=streams)
            Xd, dYd = X[perm], dY[perm]                 # the caller's row order
        else:
            plan = Plan(off, ranks, D_IN, D_OUT, "bf16", n_streams=streams)
            Xd, dYd = X, dY
        layer = PackedLoRALinear(plan, W0, [A[i] for i in active], [B[i] for i in active], scales)
        Y = layer.forward(to_dev(Xd, "bf16"))
        dX = layer.backward(to_dev(dYd, "bf16"), to_dev(Xd, "bf16"))
        torch.cuda.synchronize()
        Yh, dXh = to_host_f64(Y), to_host_f64(dX)
        if ids:
            # the oracle takes the rows grouped by adapter, in the plan's order (Z' and dZ are stored so)
            G = plan.export("perm")
            X, dY, Yh, dXh = Xd[G], dYd[G], Yh[G], dXh[G]
        out = {"Y": Yh, "dX": dXh, "dA": [to_host_f64(t) for t in layer.dA],
               "dB": [to_host_f64(t) for t in layer.dB], "Z": to_host_f64(layer.Z),
               "dZ": workspace_dz(plan, layer), "plan": plan}
        h = {"X": X, "dY": dY, "W0": W0h, "A": [Ah[i] for i in active], "B": [Bh[i] for i in active],
             "scales": np.asarray(scales, dtype=np.float32), "offsets": off, "ranks": np.asarray(ranks)}
        compare(SimpleNamespace(dtype="bf16"), h, out, what=f"replan step {k}")
