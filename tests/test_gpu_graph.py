"""Forward and backward captured in a HIP graph (torch.cuda.graph) and replayed.

The library enqueues only kernels and stream-ordering events (no memsets,
no allocations), so a caller can capture a whole step, internal streams
included.  Each case runs one eager step first (the plan creates its
internal streams then), captures forward+backward, and replays the graph
three times with new inputs copied in eagerly between replays; every replay
must equal, bit for bit, an eager step on the same inputs.  One case has one
stream group (its backward still forks the weight-gradient stream and joins
it inside the graph), one splits K.  Plans with several stream groups are
refused under capture (see the skipped case).  The per-adapter AdamW step,
with and without gradient clipping, is captured the same way and each
replay from a restored state equals the eager step."""
import numpy as np
import pytest

from tests.gpu_harness import custom_workload, say, to_dev
from workloads.tensors import host_tensors

CASES = [
    ("one stream", 256, 320, [8, 64, 3], [150, 300, 77], 1),
    pytest.param("three groups", 320, 256, [16, 200, 4, 33], [500, 9, 260, 100], 3,
                 marks=pytest.mark.skip(reason="ending the capture of a plan with several stream groups "
                                               "crashed in the runtime (torch.cuda.graph capture_end); the "
                                               "library now refuses such plans on a capturing stream")),
    ("split K", 1024, 1024, [16, 64], [200, 160], 1),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,d_in,d_out,ranks,tokens,streams", CASES)
def test_graph_replay_matches_eager(name, d_in, d_out, ranks, tokens, streams):
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    say(f"case graph {name}: {d_in}x{d_out} ranks {ranks} tokens {tokens} streams {streams}")
    w = custom_workload(name, "bf16", d_in, d_out, ranks, tokens, seed=13, n_streams=streams)
    h = host_tensors(w, 0)
    plan = Plan(h["offsets"], h["ranks"], d_in, d_out, "bf16", n_streams=streams)
    layer = PackedLoRALinear(plan, to_dev(h["W0"], "bf16"), [to_dev(a, "bf16") for a in h["A"]],
                             [to_dev(b, "bf16") for b in h["B"]], h["scales"])
    T = h["X"].shape[0]
    X = to_dev(h["X"], "bf16")
    dY = to_dev(h["dY"], "bf16")
    Y = torch.empty((T, d_out), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((T, d_in), dtype=torch.bfloat16, device="cuda")

    def step():
        layer.forward(X, Y)
        layer.backward(dY, X, dX)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                     # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    gen = torch.Generator(device="cuda").manual_seed(7)
    for rep in range(3):
        Xn = torch.randn((T, d_in), generator=gen, device="cuda").to(torch.bfloat16)
        dYn = torch.randn((T, d_out), generator=gen, device="cuda").to(torch.bfloat16)
        X.copy_(Xn)
        dY.copy_(dYn)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [Y.clone(), dX.clone()] + [t.clone() for t in layer.dA] + [t.clone() for t in layer.dB]
        step()                                     # eager on the same inputs
        torch.cuda.synchronize()
        want = [Y, dX] + list(layer.dA) + list(layer.dB)
        for k, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {rep}: output {k} differs from the eager step"
    say(f"  3 replays bit-identical to eager steps")


@pytest.mark.gpu
@pytest.mark.parametrize("clip", [False, True])
def test_adamw_step_graph_replay_matches_eager(clip):
    """The per-adapter AdamW step (with and without gradient clipping)
    captured once and replayed from a restored state: every replay equals
    the eager step from the same state, bit for bit (masters, moments and
    the bf16 copies)."""
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear, AdamW, adamw_hparams
    from workloads import optim
    say(f"case graph adamw clip={clip}")
    ranks, d_in, d_out = [8, 64, 33, 1], 256, 320
    plan = Plan(np.arange(5, dtype=np.int64) * 3, ranks, d_in, d_out, "bf16")
    A32, B32 = optim.masters(ranks, d_in, d_out, 41)
    A = [torch.from_numpy(a).cuda().to(torch.bfloat16) for a in A32]
    B = [torch.from_numpy(b).cuda().to(torch.bfloat16) for b in B32]
    layer = PackedLoRALinear(plan, None, A, B, [1.0] * len(ranks))
    opt = AdamW(layer)
    for dst, src in zip(opt.A + opt.B, A32 + B32):
        dst.copy_(torch.from_numpy(src).cuda())
    gA, gB = optim.gradients(ranks, d_in, d_out, 41, 0)
    for i in range(len(ranks)):
        layer.dA[i].copy_(torch.from_numpy(gA[i]).cuda())
        layer.dB[i].copy_(torch.from_numpy(gB[i]).cuda())
    hps = [dict(h, start=0, max_grad_norm=0.05 if i % 2 == 0 else 0.0)
           for i, h in enumerate(optim.hyperparameters(len(ranks), 41))]
    hp = adamw_hparams(optim.step_hparams(hps, 0))
    state = opt.A + opt.B + opt.mA + opt.vA + opt.mB + opt.vB + list(layer.A) + list(layer.B)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        opt.step(hp, clip_grads=clip)                 # eager warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    s0 = [t.clone() for t in state]                   # the state the graph starts from
    opt.step(hp, clip_grads=clip)
    torch.cuda.synchronize()
    want = [t.clone() for t in state]
    for t, v in zip(state, s0):
        t.copy_(v)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        opt.step(hp, clip_grads=clip)
    torch.cuda.synchronize()
    for rep in range(3):
        for t, v in zip(state, s0):
            t.copy_(v)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(state, want)):
            assert torch.equal(a, b), f"replay {rep}: state tensor {k} differs from the eager step"
    say("  3 replays bit-identical to the eager step")


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_graph_replay_with_microscaled_base(fmt):
    """Forward and backward over an MXFP8/MXFP4 base (each decodes the base
    into the workspace first) captured and replayed: every replay equals an
    eager step on the same inputs, bit for bit."""
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    from oracle import lora as ol
    from workloads.mx import pack, quantize_mx, quantize_mx4
    say(f"case graph {fmt} base")
    d_in, d_out = 512, 768
    w = custom_workload(fmt, "bf16", d_in, d_out, [16, 64], [300, 200], seed=43)
    h = host_tensors(w, 0)
    codes, scales = (quantize_mx4 if fmt == "mxfp4" else quantize_mx)(ol.as_f64(h["W0"], "bf16"), "kn")
    plan = Plan(h["offsets"], h["ranks"], d_in, d_out, "bf16", w0_format=fmt)
    layer = PackedLoRALinear(plan, torch.from_numpy(pack(codes, scales)).cuda(),
                             [to_dev(a, "bf16") for a in h["A"]], [to_dev(b, "bf16") for b in h["B"]], h["scales"])
    T = h["X"].shape[0]
    X, dY = to_dev(h["X"], "bf16"), to_dev(h["dY"], "bf16")
    Y = torch.empty((T, d_out), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((T, d_in), dtype=torch.bfloat16, device="cuda")

    def step():
        layer.forward(X, Y)
        layer.backward(dY, X, dX)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    gen = torch.Generator(device="cuda").manual_seed(44)
    for rep in range(3):
        X.copy_(torch.randn((T, d_in), generator=gen, device="cuda").to(torch.bfloat16))
        dY.copy_(torch.randn((T, d_out), generator=gen, device="cuda").to(torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [Y.clone(), dX.clone()] + [t.clone() for t in layer.dA] + [t.clone() for t in layer.dB]
        step()
        torch.cuda.synchronize()
        want = [Y, dX] + list(layer.dA) + list(layer.dB)
        for k, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {rep}: output {k} differs from the eager step"
    say("  3 replays bit-identical to eager steps")
