"""The two-layout base (w0_layout = both: [d_in][d_out] followed by its
transpose) on the GPU.

- mlora_base_transpose is exact: bf16 and fp32, square and oblong shapes,
  bit for bit against the host transpose.
- A layer over a two-layout base is bit-identical (Y, dX, every dA_i and
  dB_i, Z') to the same layer over the [d_in][d_out] base: its forward
  reads the [d_out][d_in] half and its dX the [d_in][d_out] half, and the
  GEMM's accumulation order does not depend on the operand layout.  Cases:
  segments with stream groups, split K, rows in the caller's order (ids),
  projections sharing the input, and fp32 against the oracle."""
import numpy as np
import pytest

from oracle import lora as ol
from tests.gpu_harness import TOL, custom_workload, say, to_dev, to_host_f64
from workloads.tensors import f32_to_bf16_bits, host_tensors


@pytest.mark.gpu
@pytest.mark.parametrize("dt,rows,cols", [("bf16", 192, 320), ("bf16", 4096, 4096), ("fp32", 320, 128)])
def test_base_transpose_exact(dt, rows, cols):
    import torch
    from adapter_lora_segments_amd import mlora_base_transpose
    say(f"case transpose {dt} {rows}x{cols}")
    rng = np.random.default_rng(rows + cols)
    h = rng.standard_normal((rows, cols)).astype(np.float32)
    W = to_dev(h if dt == "fp32" else f32_to_bf16_bits(h), dt)
    out = torch.empty((cols, rows), dtype=W.dtype, device="cuda")
    mlora_base_transpose(W, out)
    torch.cuda.synchronize()
    got = out.view(torch.int16 if dt == "bf16" else torch.int32).cpu().numpy()
    want = W.view(torch.int16 if dt == "bf16" else torch.int32).cpu().numpy().T
    assert np.array_equal(got, want)


def _layer_out(plan, W0, h, dt, X=None, dY=None):
    import torch
    from adapter_lora_segments_amd import PackedLoRALinear
    flat = lambda x: [v for row in x for v in row] if isinstance(x[0], list) else x
    layer = PackedLoRALinear(plan, W0, [to_dev(a, dt) for a in flat(h["A"])], [to_dev(b, dt) for b in flat(h["B"])],
                             flat(h["scales"]))
    X = to_dev(h["X"], dt) if X is None else X
    dY = to_dev(h["dY"], dt) if dY is None else dY
    Y = layer.forward(X)
    dX = layer.backward(dY, X)
    torch.cuda.synchronize()
    return [to_host_f64(Y), to_host_f64(dX), to_host_f64(layer.Z)] + [to_host_f64(t) for t in layer.dA] + \
        [to_host_f64(t) for t in layer.dB]


SEG_CASES = [
    ("three stream groups", 512, 768, [8, 64, 3, 200], [150, 300, 0, 77], 3),
    ("split K", 1024, 1024, [16, 64], [200, 160], 1),
    ("bench-like", 2048, 1024, [8, 16, 32, 64], [512, 700, 300, 900], 1),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,d_in,d_out,ranks,tokens,streams", SEG_CASES)
def test_both_layouts_bitwise_equal_to_kn(name, d_in, d_out, ranks, tokens, streams):
    from adapter_lora_segments_amd import Plan
    say(f"case two-layout base {name}: {d_in}x{d_out} ranks {ranks} tokens {tokens}")
    w = custom_workload(name, "bf16", d_in, d_out, ranks, tokens, seed=21, n_streams=streams)
    h = host_tensors(w, 0)
    W0 = to_dev(h["W0"], "bf16")
    kn = _layer_out(Plan(h["offsets"], h["ranks"], d_in, d_out, "bf16", n_streams=streams), W0, h, "bf16")
    both = _layer_out(Plan(h["offsets"], h["ranks"], d_in, d_out, "bf16", n_streams=streams, w0_layout="both"),
                      W0, h, "bf16")
    for k, (a, b) in enumerate(zip(both, kn)):
        assert np.array_equal(a, b), f"output {k} differs from the [d_in][d_out] layer"


@pytest.mark.gpu
def test_both_layouts_with_ids_and_projections():
    from adapter_lora_segments_amd import Plan
    from workloads.multi import host_multi
    say("case two-layout base with shuffled ids, then with projections sharing the input")
    w = custom_workload("ids", "bf16", 1024, 512, [8, 128, 32], [150, 260, 90], seed=22)
    h = host_tensors(w, 0)
    T = h["X"].shape[0]
    order = np.random.default_rng(3).permutation(T)
    ids = np.repeat(np.arange(3), np.diff(h["offsets"]))[order]
    h2 = dict(h, X=np.ascontiguousarray(h["X"][order]), dY=np.ascontiguousarray(h["dY"][order]))
    W0 = to_dev(h["W0"], "bf16")
    kn = _layer_out(Plan.from_ids(ids, h["ranks"], 1024, 512, "bf16"), W0, h2, "bf16")
    both = _layer_out(Plan.from_ids(ids, h["ranks"], 1024, 512, "bf16", w0_layout="both"), W0, h2, "bf16")
    for k, (a, b) in enumerate(zip(both, kn)):
        assert np.array_equal(a, b), f"ids: output {k} differs"
    widths = [512, 256]
    rk = [[8, 8], [64, 16], [100, 4]]
    hm = host_multi(23, 512, widths, rk, [300, 150, 77], "bf16")
    Wm = to_dev(hm["W0"], "bf16")
    kn = _layer_out(Plan.multi(hm["offsets"], rk, 512, widths, "bf16"), Wm, hm, "bf16")
    both = _layer_out(Plan.multi(hm["offsets"], rk, 512, widths, "bf16", w0_layout="both"), Wm, hm, "bf16")
    for k, (a, b) in enumerate(zip(both, kn)):
        assert np.array_equal(a, b), f"projections: output {k} differs"


@pytest.mark.gpu
def test_both_layouts_fp32_against_oracle():
    from adapter_lora_segments_amd import Plan
    say("case two-layout base fp32 against the oracle")
    w = custom_workload("fp32", "fp32", 256, 320, [4, 33, 8], [70, 130, 0], seed=24)
    h = host_tensors(w, 0)
    out = _layer_out(Plan(h["offsets"], h["ranks"], 256, 320, "fp32", w0_layout="both"), to_dev(h["W0"], "fp32"),
                     h, "fp32")
    off = h["offsets"]
    Yo, _ = ol.forward(h["X"], h["W0"], h["A"], h["B"], h["scales"], off, "fp32")
    dXo, dAo, dBo, _ = ol.backward(h["dY"], h["X"], h["W0"], h["A"], h["B"], h["scales"], off, "fp32")
    n = len(h["A"])
    errs = [ol.max_rel_err(out[0], Yo), ol.max_rel_err(out[1], dXo)]
    errs += [ol.max_rel_err(out[3 + i], dAo[i]) for i in range(n)]
    errs += [ol.max_rel_err(out[3 + n + i], dBo[i]) for i in range(n)]
    say(f"  worst {max(errs):.3e}")
    assert max(errs) <= TOL["fp32"]
