"""Guard bands around every buffer the library writes, on the GPU.

Each output (Y, the saved Z', dX, every dA_i and dB_i, the workspace, and for
the optimizer the fp32 masters, both moments and the bf16 copies) is a view
into a larger allocation whose bytes before and after it hold a fixed
pattern; after a forward, a backward and an AdamW step the pattern must be
intact, and the inputs (X, dY, W0, the adapters' bf16 weights before the
optimizer) must be unchanged.  A kernel that writes past its buffer, or a
launch whose grid covers more rows or columns than it should, shows up here
even when the value it writes is right.  Cases: segments with ragged row
tails and a partial output tile, three stream groups with split-K, rows as
shuffled ids, two projections sharing the input, an MXFP8 base with MXFP8
activations, fp32, and the allocation-free forward."""
import numpy as np
import pytest

from tests.gpu_harness import custom_workload, say, to_dev
from workloads.tensors import host_tensors

GUARD = 4096             # bytes on each side, a multiple of 256 so the views stay aligned
PATTERN = 0xA5


class Guarded:
    def __init__(self):
        self.bufs = []

    def tensor(self, shape, dtype, name):
        import torch
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape)) * esz
        raw = torch.full((GUARD + n + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.bufs.append((name, raw, n))
        return raw[GUARD:GUARD + n].view(dtype).view(*shape)

    def like(self, t, name):
        v = self.tensor(tuple(t.shape), t.dtype, name)
        v.copy_(t)
        return v

    def check(self, what):
        import torch
        torch.cuda.synchronize()
        bad = []
        for name, raw, n in self.bufs:
            head, tail = raw[:GUARD], raw[GUARD + n:]
            if not bool((head == PATTERN).all()) or not bool((tail == PATTERN).all()):
                bad.append(name)
        say(f"  {what}: {len(self.bufs)} guarded buffers intact" if not bad else f"  {what}: overwritten {bad}")
        assert not bad, f"{what}: guard bands overwritten around {bad}"


def _guard_layer(layer, g):
    """Replace the layer's own output buffers by guarded views."""
    from adapter_lora_segments_amd.binding import pointer_table
    import torch
    plan = layer.plan
    i = plan.info
    layer.dA = [g.tensor((i["d_in"], int(r)), torch.float32, f"dA{k}") for k, r in enumerate(plan.ranks)]
    layer.dB = [g.tensor((int(r), int(w)), torch.float32, f"dB{k}")
                for k, (r, w) in enumerate(zip(plan.ranks, plan.pair_widths))]
    layer.dA_ptrs = pointer_table(layer.dA)
    layer.dB_ptrs = pointer_table(layer.dB)
    layer.ws = g.tensor((max(1, i["workspace_bytes"]),), torch.uint8, "workspace")
    plan.upload(layer.ws)
    dt = torch.bfloat16 if plan.dtype == "bf16" else torch.float32
    layer.Z = g.tensor((max(1, i["z_elems"]),), dt, "Z")


def _guard_optimizer(opt, g):
    from adapter_lora_segments_amd.binding import pointer_table
    bf16 = opt.layer.plan.dtype == "bf16"
    if bf16:
        opt.A = [g.like(a, f"master A{k}") for k, a in enumerate(opt.A)]
        opt.B = [g.like(b, f"master B{k}") for k, b in enumerate(opt.B)]
        opt.A_ptrs, opt.B_ptrs = pointer_table(opt.A), pointer_table(opt.B)
    for nm in ("mA", "vA", "mB", "vB"):
        ts = [g.like(t, f"{nm}{k}") for k, t in enumerate(getattr(opt, nm))]
        setattr(opt, nm, ts)
        setattr(opt, nm + "_ptrs", pointer_table(ts))


def _run(plan, g, W0, A, B, scales, X, dY, T, d_in, d_out, dt, optimizer=True):
    import torch
    from adapter_lora_segments_amd import PackedLoRALinear
    from adapter_lora_segments_amd.binding import AdamW
    inputs = {"X": X.clone(), "dY": dY.clone(), "W0": W0.clone()}
    layer = PackedLoRALinear(plan, W0, A, B, scales)
    _guard_layer(layer, g)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    Y = g.tensor((T, d_out), tdt, "Y")
    dX = g.tensor((T, d_in), tdt, "dX")
    layer.forward(X, Y)
    layer.backward(dY, X, dX)
    g.check("forward + backward")
    assert bool(torch.isfinite(Y.float()).all()) and bool(torch.isfinite(dX.float()).all())
    for k, t in inputs.items():
        assert torch.equal({"X": X, "dY": dY, "W0": W0}[k], t), f"{k} was written"
    if optimizer:
        opt = AdamW(layer)
        _guard_optimizer(opt, g)
        n = len(plan.ranks)
        hp = [dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1, max_grad_norm=1.0)
              for _ in range(n)]
        opt.step(hp, clip_grads=True)
        g.check("AdamW step")
    return layer


def _adapters(h, dt, g):
    A = [g.like(to_dev(a, dt), f"A{k}") for k, a in enumerate(h["A"])]
    B = [g.like(to_dev(b, dt), f"B{k}") for k, b in enumerate(h["B"])]
    return A, B


CASES = [
    # name, dtype, d_in, d_out, ranks, tokens, streams, layout
    ("segments", "bf16", 512, 704, [8, 130, 256, 33], [300, 45, 260, 1], 1, "kn"),
    ("three groups, split-K", "bf16", 2048, 1024, [16, 64, 200, 8, 100], [70, 33, 90, 1, 60], 3, "nk"),
    ("fp32", "fp32", 256, 320, [4, 40, 17], [50, 0, 77], 2, "kn"),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,dt,d_in,d_out,ranks,tokens,streams,layout", CASES)
def test_guard_bands(name, dt, d_in, d_out, ranks, tokens, streams, layout):
    from adapter_lora_segments_amd import Plan
    say(f"case guards {name}: {dt} {d_in}x{d_out} ranks {ranks} tokens {tokens} streams {streams} {layout}")
    w = custom_workload("guards", dt, d_in, d_out, ranks, tokens, seed=4)
    h = host_tensors(w, 0)
    g = Guarded()
    T = int(h["offsets"][-1])
    plan = Plan(h["offsets"], h["ranks"], d_in, d_out, dt, n_streams=streams, w0_layout=layout)
    W0h = h["W0"] if layout == "kn" else np.ascontiguousarray(h["W0"].T)
    A, B = _adapters(h, dt, g)
    _run(plan, g, g.like(to_dev(W0h, dt), "W0"), A, B, h["scales"], g.like(to_dev(h["X"], dt), "X"),
         g.like(to_dev(h["dY"], dt), "dY"), T, d_in, d_out, dt)


@pytest.mark.gpu
def test_guard_bands_shuffled_ids():
    from adapter_lora_segments_amd import Plan
    say("case guards, rows as shuffled ids")
    w = custom_workload("guards_ids", "bf16", 768, 512, [24, 128, 64], [130, 71, 97], seed=6)
    h = host_tensors(w, 0)
    g = Guarded()
    T = int(h["offsets"][-1])
    ids = np.repeat(np.arange(3), np.diff(h["offsets"]))[np.random.default_rng(1).permutation(T)]
    plan = Plan.from_ids(ids, h["ranks"], 768, 512, "bf16", n_streams=2)
    A, B = _adapters(h, "bf16", g)
    _run(plan, g, g.like(to_dev(h["W0"], "bf16"), "W0"), A, B, h["scales"], g.like(to_dev(h["X"], "bf16"), "X"),
         g.like(to_dev(h["dY"], "bf16"), "dY"), T, 768, 512, "bf16")


@pytest.mark.gpu
def test_guard_bands_two_projections():
    from adapter_lora_segments_amd import Plan
    from workloads.multi import host_multi
    widths, ranks, tokens = [256, 512], [[8, 64], [130, 16], [256, 1]], [150, 0, 97]
    say(f"case guards, projections {widths}")
    h = host_multi(14, 512, widths, ranks, tokens, "bf16")
    g = Guarded()
    T = int(h["offsets"][-1])
    plan = Plan.multi(h["offsets"], h["ranks"], 512, widths, "bf16", n_streams=2)
    flat = lambda nested: [x for row in nested for x in row]
    A = [g.like(to_dev(a, "bf16"), f"A{k}") for k, a in enumerate(flat(h["A"]))]
    B = [g.like(to_dev(b, "bf16"), f"B{k}") for k, b in enumerate(flat(h["B"]))]
    _run(plan, g, g.like(to_dev(h["W0"], "bf16"), "W0"), A, B, flat(h["scales"]),
         g.like(to_dev(h["X"], "bf16"), "X"), g.like(to_dev(h["dY"], "bf16"), "dY"), T, 512, sum(widths), "bf16")


@pytest.mark.gpu
def test_guard_bands_mxfp8_activations():
    import torch
    from adapter_lora_segments_amd import Plan
    from workloads.mx import quantize_mx_device
    say("case guards, MXFP8 base with MXFP8 activations")
    w = custom_workload("guards_mx", "bf16", 1024, 768, [32, 200, 8], [100, 130, 3], seed=7)
    h = host_tensors(w, 0)
    g = Guarded()
    T = int(h["offsets"][-1])
    plan = Plan(h["offsets"], h["ranks"], 1024, 768, "bf16", w0_layout="nk", w0_format="mxfp8", act_format="mxfp8")
    packed = quantize_mx_device(to_dev(h["W0"], "bf16"), "nk")
    A, B = _adapters(h, "bf16", g)
    _run(plan, g, g.like(packed, "W0 codes"), A, B, h["scales"], g.like(to_dev(h["X"], "bf16"), "X"),
         g.like(to_dev(h["dY"], "bf16"), "dY"), T, 1024, 768, "bf16", optimizer=False)
    assert packed.dtype == torch.uint8


@pytest.mark.gpu
def test_guard_bands_allocation_free_forward():
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    from adapter_lora_segments_amd.binding import mlora_forward_noalloc
    say("case guards, allocation-free forward")
    w = custom_workload("guards_na", "bf16", 512, 512, [16, 256], [90, 77], seed=3)
    h = host_tensors(w, 0)
    g = Guarded()
    T = int(h["offsets"][-1])
    plan = Plan(h["offsets"], h["ranks"], 512, 512, "bf16")
    A, B = _adapters(h, "bf16", g)
    layer = PackedLoRALinear(plan, g.like(to_dev(h["W0"], "bf16"), "W0"), A, B, h["scales"])
    X = g.like(to_dev(h["X"], "bf16"), "X")
    Y = g.tensor((T, 512), torch.bfloat16, "Y")
    Z = g.tensor((max(1, plan.info["z_elems"]),), torch.bfloat16, "Z")
    for _ in range(2):
        mlora_forward_noalloc(plan, X, layer.W0, layer.A_ptrs, layer.B_ptrs, layer.scales, Y, Z)
    g.check("allocation-free forward")
