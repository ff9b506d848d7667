"""mlora_forward_noalloc, the forward for callers that cannot allocate: the
same kernels in the same order as mlora_forward, with the work buffers in
the library's static scratch instead of a caller workspace.

On the GPU, through the C interface: calls in a row on one device (the
scratch keeps the previous call's contents), each equal bit for bit to
mlora_forward on the same inputs and within the oracle's bar; the second
call's input is smaller than the first's.  Cases cover both W0 layouts (the
[d_out][d_in] base reads B_cat^T from the scratch), split-K partial tiles,
two stream groups, and fp32.  On the host: a layer whose buffers exceed the
scratch is refused before any device call."""
import ctypes

import numpy as np
import pytest

from adapter_lora_segments_amd import _lib
from adapter_lora_segments_amd.binding import Plan


def test_noalloc_refuses_layers_beyond_the_scratch_without_launching():
    # rank-padded A_cat^T alone: 8 adapters x r_pad 256 x d_in 16384 x 2 bytes = 64 MiB, plus the tables
    p = Plan(np.arange(9, dtype=np.int64) * 4, [256] * 8, 16384, 1024)
    vp = ctypes.c_void_p
    dummy = vp(1 << 20)
    L = _lib.lib()
    assert L.mlora_forward_noalloc(p.handle, dummy, dummy, dummy, dummy, dummy, dummy, dummy, None) == -2
    msg = L.mlora_last_error().decode()
    assert "scratch" in msg and str(64 << 20) in msg
    assert L.mlora_forward_noalloc(p.handle, None, dummy, dummy, dummy, dummy, dummy, dummy, None) == -1
    assert L.mlora_forward_noalloc(p.handle, vp((1 << 20) + 4), dummy, dummy, dummy, dummy, dummy, dummy,
                                   None) == -1


# (dtype, d_in, d_out, ranks, tokens, streams, layout): input sizes T x d_in decrease from case to case
CASES = [
    ("bf16", 1024, 1536, [8, 64, 3, 200], [300, 900, 0, 450], 2, "nk"),
    ("bf16", 2048, 2048, [16, 64], [200, 312], 1, "kn"),        # 512 rows: split-K partial tiles
    ("bf16", 256, 320, [8, 64, 4], [150, 300, 1], 1, "kn"),
    ("fp32", 256, 256, [4, 8], [64, 64], 1, "nk"),
]


@pytest.mark.gpu
def test_noalloc_forward_matches_forward_call_after_call():
    import torch
    from adapter_lora_segments_amd import PackedLoRALinear, mlora_forward, mlora_forward_noalloc
    from oracle import lora as ol
    from tests.gpu_harness import TOL, custom_workload, say, to_dev, to_host_f64
    from workloads.tensors import host_tensors
    sizes = [t * d for (_, d, _, _, tok, _, _) in CASES for t in [sum(tok)]]
    assert sizes == sorted(sizes, reverse=True)
    for k, (dt, d_in, d_out, ranks, tokens, streams, layout) in enumerate(CASES):
        say(f"case noalloc {k}: {dt} {d_in}x{d_out} ranks {ranks} tokens {tokens} streams {streams} {layout}")
        w = custom_workload(f"noalloc{k}", dt, d_in, d_out, ranks, tokens, seed=31 + k, n_streams=streams)
        h = host_tensors(w, 0)
        plan = Plan(h["offsets"], h["ranks"], d_in, d_out, dt, n_streams=streams, w0_layout=layout)
        W0h = h["W0"] if layout == "kn" else np.ascontiguousarray(h["W0"].T)
        layer = PackedLoRALinear(plan, to_dev(W0h, dt), [to_dev(a, dt) for a in h["A"]],
                                 [to_dev(b, dt) for b in h["B"]], h["scales"])
        X = to_dev(h["X"], dt)
        T = X.shape[0]
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        Y1 = torch.full((T, d_out), float("nan"), dtype=tdt, device="cuda")
        Y2 = torch.full((T, d_out), float("nan"), dtype=tdt, device="cuda")
        Z1 = plan.alloc_z().fill_(float("nan"))
        Z2 = plan.alloc_z().fill_(float("nan"))
        mlora_forward(plan, X, layer.W0, layer.A_ptrs, layer.B_ptrs, layer.scales, Y1, Z1, layer.ws)
        mlora_forward_noalloc(plan, X, layer.W0, layer.A_ptrs, layer.B_ptrs, layer.scales, Y2, Z2)
        torch.cuda.synchronize()
        assert torch.equal(Y1, Y2), f"case {k}: Y differs from mlora_forward"
        assert torch.equal(Z1[:plan.info["z_elems"]], Z2[:plan.info["z_elems"]]), f"case {k}: Z differs"
        Y, _ = ol.forward(h["X"], h["W0"], h["A"], h["B"], h["scales"], h["offsets"], dt)
        e = ol.max_rel_err(to_host_f64(Y2), Y)
        say(f"  bit-identical to mlora_forward; Y against the oracle {e:.3e}")
        assert e <= TOL[dt]
