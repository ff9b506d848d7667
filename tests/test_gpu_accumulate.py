"""Gradient accumulation (plan option grad_accumulate) on the GPU.

A plan with grad_accumulate adds each backward's dA_i and dB_i to what the
gradient buffers hold.  Checked bit for bit against the same plan without it:
starting from arbitrary values G, one accumulating backward must give exactly
G + (the overwriting backward's gradients), one fp32 rounding of the sum,
whichever path wrote them (a single-chunk adapter's direct write, the
fixed-order sum of several chunks' partials, the fp32 kernels); an adapter
with no rows keeps G; a second accumulating backward adds again.  Over
segments and shuffled ids, one and three stream groups, the weight gradients
beside and after the dX GEMM, bf16 and fp32."""
import numpy as np
import pytest

from tests.gpu_harness import custom_workload, say, to_dev
from workloads.tensors import host_tensors

CASES = [
    # name, dtype, d_in, d_out, ranks, tokens (3000 rows of rank 8: 12 chunks; 100 rows: one chunk;
    # an adapter with no rows), streams, wg_overlap, ids
    ("segments", "bf16", 512, 768, [8, 64, 256, 16], [3000, 100, 0, 700], 1, "auto", False),
    ("three groups, after", "bf16", 512, 512, [8, 130, 33, 16], [2000, 64, 0, 900], 3, "after", False),
    ("shuffled ids", "bf16", 256, 512, [8, 200, 16], [1500, 40, 300], 2, "auto", True),
    ("fp32", "fp32", 256, 320, [4, 40, 17], [300, 0, 77], 1, "auto", False),
]


def _layer(h, dt, plan):
    from adapter_lora_segments_amd import PackedLoRALinear
    return PackedLoRALinear(plan, to_dev(h["W0"], dt), [to_dev(a, dt) for a in h["A"]],
                            [to_dev(b, dt) for b in h["B"]], h["scales"])


@pytest.mark.gpu
@pytest.mark.parametrize("name,dt,d_in,d_out,ranks,tokens,streams,wg,ids", CASES)
def test_accumulating_backward_adds_exactly(name, dt, d_in, d_out, ranks, tokens, streams, wg, ids):
    import torch
    from adapter_lora_segments_amd import Plan
    say(f"case accumulate {name}: {dt} {d_in}x{d_out} ranks {ranks} tokens {tokens} streams {streams} wg {wg}")
    w = custom_workload("accumulate", dt, d_in, d_out, ranks, tokens, seed=12)
    h = host_tensors(w, 0)
    T = int(h["offsets"][-1])
    opts = dict(n_streams=streams, wg_overlap=wg)
    if ids:
        tok = np.repeat(np.arange(len(ranks)), tokens)[np.random.default_rng(4).permutation(T)]
        mk = lambda acc: Plan.from_ids(tok, h["ranks"], d_in, d_out, dt, grad_accumulate=acc, **opts)
    else:
        mk = lambda acc: Plan(h["offsets"], h["ranks"], d_in, d_out, dt, grad_accumulate=acc, **opts)
    over, accu = _layer(h, dt, mk(False)), _layer(h, dt, mk(True))
    X, dY = to_dev(h["X"], dt), to_dev(h["dY"], dt)
    dY2 = to_dev(np.ascontiguousarray(h["dY"][::-1]), dt)
    g = torch.Generator(device="cuda").manual_seed(5)
    G_A = [torch.randn(t.shape, generator=g, device="cuda") for t in accu.dA]
    G_B = [torch.randn(t.shape, generator=g, device="cuda") for t in accu.dB]
    for t, v in zip(accu.dA + accu.dB, G_A + G_B):
        t.copy_(v)
    over.forward(X)
    accu.forward(X)
    dX_o = over.backward(dY, X)
    dX_a = accu.backward(dY, X)
    torch.cuda.synchronize()
    assert torch.equal(dX_o, dX_a), "dX differs between the two plans"
    for i in range(len(ranks)):
        assert torch.equal(accu.dA[i], G_A[i] + over.dA[i]), f"dA {i} is not G + the overwritten gradient"
        assert torch.equal(accu.dB[i], G_B[i] + over.dB[i]), f"dB {i} is not G + the overwritten gradient"
        if tokens[i] == 0:
            assert torch.equal(accu.dA[i], G_A[i]) and torch.equal(accu.dB[i], G_B[i]), f"empty adapter {i} changed"
            assert not bool(over.dA[i].any()) and not bool(over.dB[i].any()), f"empty adapter {i} not zeroed"
    # a second micro-batch adds again
    first_A = [t.clone() for t in accu.dA]
    first_B = [t.clone() for t in accu.dB]
    over.backward(dY2, X)
    accu.backward(dY2, X)
    torch.cuda.synchronize()
    for i in range(len(ranks)):
        assert torch.equal(accu.dA[i], first_A[i] + over.dA[i]), f"second step: dA {i}"
        assert torch.equal(accu.dB[i], first_B[i] + over.dB[i]), f"second step: dB {i}"
    say(f"  {2 * len(ranks)} gradients: G + overwritten, bit for bit, over two micro-batches")
