"""Seeded tensor values for a workload projection.

Host path (numpy): values drawn in fp32 from ``default_rng(SeedSequence(...))``
and, in bf16 workloads, rounded to bf16 with round-to-nearest-even; bf16
tensors are returned as ``uint16`` bit patterns.  The same bits go to the
oracle (upcast to fp64) and to the device.

Device path (torch, for the large workloads that do not fit a reasonable host
budget): ``torch.randn`` with a seeded ``torch.Generator`` on the device, scaled
and converted to bf16 by torch (also round-to-nearest-even).  Rows the oracle
needs are copied back to the host.  Neither path holds any of the layer's
arithmetic.
"""
from __future__ import annotations

import numpy as np

from .configs import Workload, STD_X, STD_DY, STD_W0, STD_B, std_a

_TENSOR_IDS = {"X": 1, "W0": 2, "A": 3, "B": 4, "dY": 5}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, proj: int, tensor: str, idx: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, proj, _TENSOR_IDS[tensor], idx]))


def _draw(rng, shape, std, dtype):
    v = rng.standard_normal(size=shape, dtype=np.float32)
    v *= np.float32(std)
    if dtype == "bf16":
        return f32_to_bf16_bits(v)
    return v


def host_tensors(w: Workload, proj: int = 0, seed: int | None = None,
                 b_zero: bool = False, rows: int | None = None) -> dict:
    """All inputs of projection ``proj`` as host arrays.

    Returns dict with X [T,d_in], W0 [d_in,d_out], A list of [d_in,r_i],
    B list of [r_i,d_out], dY [T,d_out], scales (float32 [n]), offsets
    (int64 [n+1]), ranks (int32 [n]).  bf16 tensors are uint16 bit arrays.
    With ``rows`` only the first ``rows`` tokens are drawn (the same values
    as the full tensors' leading rows; the generator fills row by row) and
    the offsets are cut there.
    """
    s = w.seed if seed is None else seed
    p = w.projections[proj]
    dt = w.dtype
    T = w.T if rows is None else min(int(rows), w.T)
    out = {
        "X": _draw(_rng(s, proj, "X"), (T, p.d_in), STD_X, dt),
        "W0": _draw(_rng(s, proj, "W0"), (p.d_in, p.d_out), STD_W0, dt),
        "dY": _draw(_rng(s, proj, "dY"), (T, p.d_out), STD_DY, dt),
        "A": [_draw(_rng(s, proj, "A", i), (p.d_in, r), std_a(p.d_in), dt) for i, r in enumerate(w.ranks)],
        "B": [(_draw(_rng(s, proj, "B", i), (r, p.d_out), STD_B, dt) if not b_zero else
               np.zeros((r, p.d_out), dtype=np.uint16 if dt == "bf16" else np.float32))
              for i, r in enumerate(w.ranks)],
        "scales": np.asarray(w.scales, dtype=np.float32),
        "offsets": np.minimum(w.seg_offsets(), T),
        "ranks": np.asarray(w.ranks, dtype=np.int32),
        "dtype": dt,
        "d_in": p.d_in,
        "d_out": p.d_out,
    }
    return out


def device_tensors(w: Workload, proj: int = 0, seed: int | None = None, device: str = "cuda",
                   sets: int = 1):
    """Inputs drawn on the device with torch (bf16 workloads only).

    ``sets`` > 1 draws that many independent (X, dY) pairs sharing W0, A, B,
    for benchmarks that rotate activations.  Returns dict of torch tensors.
    """
    import torch

    s = w.seed if seed is None else seed
    p = w.projections[proj]
    T = w.T
    assert w.dtype == "bf16"

    def gen(tid, idx=0):
        g = torch.Generator(device=device)
        g.manual_seed((s * 1000003 + proj * 7919 + _TENSOR_IDS[tid] * 104729 + idx * 31) & 0x7FFFFFFF)
        return g

    def draw(shape, std, tid, idx=0):
        t = torch.randn(shape, generator=gen(tid, idx), device=device, dtype=torch.float32)
        t.mul_(std)
        return t.to(torch.bfloat16)

    out = {
        "W0": draw((p.d_in, p.d_out), STD_W0, "W0"),
        "A": [draw((p.d_in, r), std_a(p.d_in), "A", i) for i, r in enumerate(w.ranks)],
        "B": [draw((r, p.d_out), STD_B, "B", i) for i, r in enumerate(w.ranks)],
        "X": [draw((T, p.d_in), STD_X, "X", k) for k in range(sets)],
        "dY": [draw((T, p.d_out), STD_DY, "dY", k) for k in range(sets)],
        "scales": np.asarray(w.scales, dtype=np.float32),
        "offsets": w.seg_offsets(),
        "ranks": np.asarray(w.ranks, dtype=np.int32),
        "dtype": "bf16",
        "d_in": p.d_in,
        "d_out": p.d_out,
    }
    return out
