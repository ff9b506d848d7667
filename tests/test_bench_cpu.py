"""Host logic of bench.py (no GPU): the one-GPU refusal and the algorithmic
byte and FLOP counts behind the roofline fields."""
import subprocess
import sys

import pytest

import bench
from workloads import load_workload


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _fake(ms=1.0, n=1):
    kinds = ["shrink", "gemm_fwd", "dz", "token_reduce", "reduce", "gemm_dx", "prep", "adamw", "dequant",
             "grad_norm"]
    return {k: (ms, n) for k in kinds}


@pytest.mark.parametrize("fmt,code_bytes", [("mxfp8", 1.0), ("mxfp4", 0.5)])
def test_dequant_bytes_per_weight(fmt, code_bytes):
    """Two decodes a step, each reading the codes and 1/32 byte of scales and
    writing 2 bytes per weight: at 1 ms per step the rate is those bytes per ms."""
    w = load_workload("llama7b_proj", 0)
    p = w.projections[0]
    out = bench.kernel_rooflines(w, [[0]], _fake(), _fake(), 1, fmt)
    want = 2 * (code_bytes + 1 / 32 + 2) * p.d_in * p.d_out / 1e-3 / 1e9
    assert out["dequant"]["achieved"] == pytest.approx(want)


def test_gemm_flops_count_base_and_lora_term():
    """Forward GEMM: 2 T d_in d_out base flops plus 2 sum(n_i r_i) d_out for
    the fused expand; at 1 ms the TFLOP/s figure is that count / 1e9."""
    w = load_workload("llama7b_proj", 0)
    p = w.projections[0]
    snr = sum(n * r for n, r in zip(w.tokens, w.ranks))
    out = bench.kernel_rooflines(w, [[0]], _fake(), _fake(), 1)
    want = (2.0 * w.T * p.d_in * p.d_out + 2.0 * snr * p.d_out) / 1e-3 / 1e12
    assert out["gemm_fwd"]["achieved"] == pytest.approx(want)
    assert out["gemm_fwd"]["bound"] == "mfma" and out["shrink"]["bound"] == "hbm"
