"""HIP path against the oracle, element by element, through the C interface.

Tolerances (max |g - o| / max |o| per output tensor, per adapter for dA_i,
dB_i and the saved Z'_i): 2e-2 in bf16 mode, 1e-4 in fp32 mode."""
import numpy as np
import pytest

from tests.gpu_harness import custom_workload, run_gpu, compare, say
from workloads import load_workload

pytestmark = pytest.mark.gpu


def test_device_is_gfx950():
    from adapter_lora_segments_amd import device_check
    device_check()


def test_tiny_fp32_workload():
    w = load_workload("tiny_fp32", 0)
    say("case tiny_fp32 seed 0")
    h, out = run_gpu(w)
    compare(w, h, out, what="tiny_fp32")


@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_fp32_ragged_multi_tile(layout):
    # several 64-row GEMM tiles, ragged tail, empty and one-row adapters,
    # ranks not multiples of 8, K not a multiple of 256
    w = custom_workload("fp32_ragged", "fp32", 192, 320, [4, 7, 1, 33, 256, 16],
                        [130, 0, 1, 77, 200, 5], seed=3)
    say(f"case fp32_ragged layout {layout}")
    h, out = run_gpu(w, w0_layout=layout)
    compare(w, h, out, what=f"fp32_ragged_{layout}")


@pytest.mark.parametrize("name", ["llama7b_proj", "llama3_8b_layer", "nano_stress", "mlp70b_pair"])
def test_fp32_reduced_workloads(name):
    """fp32 runs of the bf16 workloads' adapter/rank structure at reduced
    token counts and dims, so LoRA-only mistakes cannot hide under bf16
    tolerance."""
    w = load_workload(name, 0)
    p = w.projections[-1]
    small = custom_workload(name + "_fp32", "fp32", min(p.d_in, 512), min(p.d_out, 448), w.ranks,
                            w.scaled_down(768).tokens, seed=1)
    say(f"case fp32 reduced {name}: T={small.T}")
    h, out = run_gpu(small)
    compare(small, h, out, what=f"{name}_fp32_reduced")


BF16_CASES = {
    # several 256-row tiles and 64-row steps, ragged tails in rows and columns,
    # empty / one-row adapters, ranks 1..256 incl. non-multiples of 8
    "ragged": ("bf16", 512, 320, [4, 7, 1, 33, 256, 16, 64], [300, 0, 1, 77, 512, 5, 190]),
    # K not a multiple of 256 (skinny remainder loop), N < 256
    "narrow": ("bf16", 192, 128, [8, 128], [97, 260]),
    # many tiny adapters sharing GEMM tiles
    "crowded": ("bf16", 256, 512, [4, 256, 8, 128, 16, 64, 32, 200, 3, 100] * 3,
                [1, 2, 3, 1, 7, 30, 1, 64, 2, 9] * 3),
}


@pytest.mark.parametrize("case", sorted(BF16_CASES))
@pytest.mark.parametrize("layout", ["kn", "nk"])
def test_bf16_small(case, layout):
    dt, d_in, d_out, ranks, toks = BF16_CASES[case]
    w = custom_workload("bf16_" + case, dt, d_in, d_out, ranks, toks, seed=5)
    say(f"case bf16 {case} layout {layout}")
    h, out = run_gpu(w, w0_layout=layout)
    compare(w, h, out, what=f"bf16_{case}_{layout}")


@pytest.mark.parametrize("streams", [2, 3, 4])
def test_bf16_stream_groups(streams):
    w = custom_workload("bf16_streams", "bf16", 256, 384, [16, 64, 8, 128, 32, 256, 4],
                        [200, 90, 300, 0, 45, 260, 17], seed=7)
    say(f"case bf16 streams {streams}")
    h, out = run_gpu(w, n_streams=streams)
    compare(w, h, out, what=f"bf16_streams{streams}")


def test_bf16_scales_zero_and_negative():
    w = custom_workload("bf16_scales", "bf16", 256, 256, [16, 32, 8], [100, 120, 70],
                        scales=[0.0, -3.0, 0.5], seed=9)
    say("case bf16 scales 0/-3/0.5")
    h, out = run_gpu(w)
    compare(w, h, out, what="bf16_scales")
    assert np.all(out["dB"][0] == 0.0) and np.all(out["dA"][0] == 0.0)


@pytest.mark.parametrize("nano_rows", [32, 64, 96, 160, 256])
def test_bf16_long_nano_batches(nano_rows):
    # nano-batches of one, two and four 32-row fragments, the last one
    # partial, and (160, 256) of several 128-row blocks; K = 320 and 192, five
    # and three 64-deep stages in the two skinny products
    w = custom_workload("bf16_nano", "bf16", 320, 192, [8, 128, 256, 32], [150, 70, 297, 33], seed=13)
    say(f"case bf16 nano_rows {nano_rows}")
    h, out = run_gpu(w, nano_rows=nano_rows)
    compare(w, h, out, what=f"bf16_nano{nano_rows}")


def test_bf16_small_chunks_many_partials():
    # tiny reduction chunks: many partial sums per adapter
    w = custom_workload("bf16_chunks", "bf16", 256, 256, [32, 64], [700, 333], seed=11)
    say("case bf16 small chunks")
    h, out = run_gpu(w, chunk_min=16, chunk_max=64, chunk_per_rank=1)
    compare(w, h, out, what="bf16_small_chunks")


def test_empty_rows_zero_gradients():
    for dt in ("bf16", "fp32"):
        w = custom_workload("empty", dt, 128, 128, [8, 16], [0, 0], seed=2)
        say(f"case empty {dt}")
        h, out = run_gpu(w)
        assert out["Y"].shape == (0, 128)
        for i in range(2):
            assert np.all(out["dA"][i] == 0.0) and np.all(out["dB"][i] == 0.0)


def test_backward_without_dx():
    w = custom_workload("nodx", "bf16", 256, 192, [16, 8], [90, 40], seed=4)
    h, out = run_gpu(w, want_dx=False)
    compare(w, h, out, what="bf16_no_dx")


def test_bitwise_repeatable():
    import torch
    w = custom_workload("repeat", "bf16", 512, 512, [64, 16, 256], [600, 257, 300], seed=6)
    say("case bitwise repeat")
    h, out = run_gpu(w)
    layer, d = out["layer"], out["dev"]
    Y1 = d["Y"].clone()
    dX1 = d["dX"].clone()
    dA1 = [t.clone() for t in layer.dA]
    dB1 = [t.clone() for t in layer.dB]
    Y2 = layer.forward(d["X"])
    dX2 = layer.backward(d["dY"], d["X"])
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2) and torch.equal(dX1, dX2)
    for a, b in zip(dA1, layer.dA):
        assert torch.equal(a, b)
    for a, b in zip(dB1, layer.dB):
        assert torch.equal(a, b)


@pytest.mark.parametrize("streams", [1, 3])
def test_weight_gradients_beside_or_after_dx(streams):
    """The backward's weight gradients on the side stream beside the dX GEMM
    and on the caller's stream after it: the same kernels on the same data,
    so every output is bitwise identical, and within the bar of the oracle."""
    w = custom_workload("placement", "bf16", 512, 768, [64, 16, 256, 8], [600, 257, 300, 33], seed=8)
    say(f"case weight gradients beside or after the dX GEMM, {streams} stream group(s)")
    res = {}
    for mode in ("side", "after"):
        h, out = run_gpu(w, wg_overlap=mode, n_streams=streams)
        assert out["plan"].info["wg_side"] == (1 if mode == "side" else 0)
        compare(w, h, out, what=f"bf16_wg_{mode}")
        res[mode] = out
    for k in ("Y", "dX", "Z", "dZ"):
        assert np.array_equal(res["side"][k], res["after"][k]), k
    for k in ("dA", "dB"):
        for a, b in zip(res["side"][k], res["after"][k]):
            assert np.array_equal(a, b), k


def test_llama7b_proj_full_size():
    """The 4096x4096 workload at full size, every output element checked."""
    w = load_workload("llama7b_proj", 0)
    say("case llama7b_proj full")
    h, out = run_gpu(w)
    compare(w, h, out, what="llama7b_proj")


def test_profile_mask_selects_kernels():
    import torch
    w = custom_workload("prof", "bf16", 256, 256, [16, 64], [100, 140], seed=3)
    say("case profile mask")
    h, out = run_gpu(w)
    layer, d = out["layer"], out["dev"]
    plan = layer.plan
    plan.profile_enable(["gemm_fwd"])
    plan.profile_read()
    layer.forward(d["X"])
    layer.backward(d["dY"], d["X"])
    torch.cuda.synchronize()
    r = plan.profile_read()
    assert r["gemm_fwd"][1] == plan.info["n_groups"] and r["gemm_fwd"][0] > 0.0
    assert all(cnt == 0 for k, (ms, cnt) in r.items() if k != "gemm_fwd")
    plan.profile_enable(True)
    layer.forward(d["X"])
    layer.backward(d["dY"], d["X"])
    torch.cuda.synchronize()
    r = plan.profile_read()
    plan.profile_enable(False)
    # every kind the forward and backward of a bf16 base launch (the optimizer
    # step is a call of its own; only an MXFP8 base is decoded, and only
    # MXFP8 activations are quantized)
    idle = ("adamw", "dequant", "grad_norm", "quant_act")
    assert all(cnt > 0 for k, (ms, cnt) in r.items() if k not in idle), r
    assert all(r[k][1] == 0 for k in idle), r
