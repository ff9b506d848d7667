"""Benchmark: packed multi-LoRA linear forward+backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one forward (shrink, base GEMM with fused expand) and one backward
(dZ, dB, dA, reduction, dX GEMM with fused dZ.A^T) of the whole layer over
one batch, on inputs already resident in device memory.  Four independent
(X, dY) sets rotate across steps so activations do not stay in the 256 MB
last-level cache.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def alg_flops(w, proj):
    """Algorithmic FLOPs of forward+backward: sum_i n_i (4 d_in d_out + 6 r_i (d_in + d_out))."""
    p = w.projections[proj]
    return sum(n * (4 * p.d_in * p.d_out + 6 * r * (p.d_in + p.d_out))
               for n, r in zip(w.tokens, w.ranks))


def gemm_fwd_flops(w, proj):
    """One forward GEMM launch: base X.W0 plus the fused expand Z'.B."""
    p = w.projections[proj]
    return 2 * w.T * p.d_in * p.d_out + sum(2 * n * r * p.d_out for n, r in zip(w.tokens, w.ranks))


GEMM_SOURCES = ("kernels_gemm.hip", "gemm_common.hpp", "device_common.hpp")


def gemm_source_hash() -> str:
    """First 16 hex digits of the sha256 of the bf16 GEMM's source files
    (the kernel file and the headers it includes, in that order), the key
    under which measured counters are stored."""
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, "adapter_lora_segments_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, layout: str = "kn"):
    """HBM bytes per forward-GEMM launch from the committed counter summary
    (profiles/hbm_bytes_<workload>.txt), or None when that file is missing,
    covers another W0 layout, or was taken from a different version of the
    kernel source."""
    if layout != "kn":
        return None
    path = os.path.join(ROOT, "profiles", f"hbm_bytes_{workload}.txt")
    if not os.path.exists(path):
        return None
    sha = gemm_source_hash()
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("gemm_sources_sha256_16") != sha:
        return None
    v = vals.get("traffic_bytes k_gemm_fwd")
    return int(v) if v else None


def kernel_rooflines(w, units, kern, iso, steps, w0_format="bf16", act_format="bf16"):
    """Achieved rate of every step of the path against its roofline, from the
    per-kernel pass (the weight-gradient kernels from the isolated pass,
    where they do not share the chip with the dX GEMM).  Algorithmic bytes
    and FLOPs count each operand once (ranks unpadded); ``units`` lists the
    projections of each timed layer, and projections in one unit share X,
    which is then counted once."""
    T = w.T
    snr = sum(n * r for n, r in zip(w.tokens, w.ranks))
    sr = sum(w.ranks)
    work = {"shrink": 0.0, "dz": 0.0, "token_reduce": 0.0, "gemm_fwd": 0.0, "gemm_dx": 0.0}
    for unit in units:
        di = w.projections[unit[0]].d_in
        P = len(unit)
        work["shrink"] += 2.0 * (T * di + P * (di * sr + snr))
        work["token_reduce"] += 2.0 * T * di + P * (2.0 * snr + 4.0 * di * sr)
        for q in unit:
            do = w.projections[q].d_out
            work["dz"] += 2.0 * (T * do + sr * do + snr)
            work["token_reduce"] += 2.0 * (T * do + snr) + 4.0 * sr * do
            work["gemm_fwd"] += 2.0 * T * di * do + 2.0 * snr * do
            work["gemm_dx"] += 2.0 * T * di * do + 2.0 * snr * di
    out = {}
    for k, src, bound in (("shrink", kern, "hbm"), ("dz", kern, "hbm"), ("token_reduce", iso, "hbm"),
                          ("gemm_fwd", kern, "mfma"), ("gemm_dx", kern, "mfma")):
        ms = src[k][0] / steps
        if ms <= 0:
            continue
        if bound == "hbm":
            ach = work[k] / (ms * 1e-3) / 1e9
            out[k] = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                      "frac": ach / PEAK_HBM_GBS, "ms_per_step": ms}
        else:
            ach = work[k] / (ms * 1e-3) / 1e12
            # the forward's base product on MXFP8 operands takes the fp8 peak
            peak = PEAK_FP8_TFLOPS if (k == "gemm_fwd" and act_format == "mxfp8") else PEAK_BF16_TFLOPS
            out[k] = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                      "frac": ach / peak, "ms_per_step": ms}
    out["gemm_dx"]["note"] = "timed beside the concurrent weight-gradient kernels"
    if kern.get("dequant", (0.0, 0))[1]:
        # microscaled base: codes (1 B for MXFP8, 0.5 B for MXFP4) and scales (1/32 B) read, bf16 (2 B)
        # written per weight, once per decode (two a step, one with MXFP8 activations)
        code_b = 0.5 if w0_format == "mxfp4" else 1.0
        per_step = 1 if act_format == "mxfp8" else 2
        byt = sum(per_step * (code_b + 1 / 32 + 2) * w.projections[q[0]].d_in * w.projections[q[0]].d_out
                  for q in units)
        ms = kern["dequant"][0] / steps
        ach = byt / (ms * 1e-3) / 1e9
        out["dequant"] = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                          "frac": ach / PEAK_HBM_GBS, "ms_per_step": ms}
    if kern.get("quant_act", (0.0, 0))[1]:
        # activations to MXFP8: 2 B read, 1 + 1/32 B written per input
        byt = sum((2 + 1 + 1 / 32) * w.T * w.projections[q[0]].d_in for q in units)
        ms = kern["quant_act"][0] / steps
        ach = byt / (ms * 1e-3) / 1e9
        out["quant_act"] = {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": ach / PEAK_HBM_GBS, "ms_per_step": ms}
    for k in ("reduce", "prep"):
        out[k] = {"bound": "overhead", "ms_per_step": iso[k][0] / steps}
    return out


def _oracle_step_seconds(w, projs):
    """One oracle forward+backward over every listed projection of ``w``
    (host tensors drawn first, not timed)."""
    from oracle import lora as ol
    from workloads.tensors import host_tensors
    dt = 0.0
    for q in projs:
        h = host_tensors(w, q)
        t0 = time.perf_counter()
        ol.forward(h["X"], h["W0"], h["A"], h["B"], h["scales"], h["offsets"], w.dtype)
        ol.backward(h["dY"], h["X"], h["W0"], h["A"], h["B"], h["scales"], h["offsets"], w.dtype)
        dt += time.perf_counter() - t0
    return dt


def cpu_baseline(w, projs, flop_budget=1.0e13):
    """The oracle (numpy float64) on the host over a bounded sample of the
    workload: the same layer shapes, adapters and ranks with every adapter's
    token count scaled down in proportion (at least one token each), chosen
    so the sample is about ``flop_budget`` floating-point operations (5e12
    took 6.8 s on 16 host threads); the whole workload when it is smaller.  Beside it, the oracle
    on one thread on the two smallest workloads (the fp32 256x256 layer
    whole, and the 4096x4096 layer on 1024 sampled tokens)."""
    from workloads import load_workload
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:
        threadpool_limits = None
        threads = os.cpu_count()
    per_token = sum(4.0 * w.projections[q].d_in * w.projections[q].d_out for q in projs)
    M = int(min(w.T, max(256, flop_budget // per_token)))
    sample = w.scaled_down(M)
    dt = _oracle_step_seconds(sample, projs)
    what = "the whole workload" if sample.T == w.T else \
        f"{sample.T} of {w.T} tokens (every adapter's tokens scaled by {M}/{w.T}, at least one each)"
    out = {"value": sample.T / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"one forward+backward of {what} over {len(projs)} projection(s) "
                     f"in float64 numpy, {dt:.2f} s"}
    if threadpool_limits is not None:
        one = {}
        with threadpool_limits(limits=1):
            for name, rows in (("tiny_fp32", None), ("llama7b_proj", 1024)):
                wl = load_workload(name, 0)
                if rows:
                    wl = wl.scaled_down(rows)
                t = _oracle_step_seconds(wl, [0])
                one[name] = {"value": wl.T / t, "unit": "tokens/s", "tokens": wl.T, "seconds": t}
        out["one_thread"] = one
    return out


def ceilings(random_only=False):
    """Measured ceilings of this GPU (libmlora_probes.so): the pure-MFMA loop
    in the base GEMM's instruction pattern with random and with zero bf16
    operands (TFLOP/s), streaming copy and read bandwidth (GB/s), and the
    rate at which L2-resident operand blocks reach LDS by the base GEMM's
    direct-to-LDS copies, by register-staged copies, and into registers only
    (GB/s, and per CU), each the best of several timed launches on torch's
    current stream."""
    import ctypes
    import torch
    from adapter_lora_segments_amd import _lib
    path = os.path.join(os.path.dirname(_lib.LIB_PATH), "libmlora_probes.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing; build it with `python -m adapter_lora_segments_amd.build`")
    L = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    L.mlora_probe_mfma.argtypes = [i64, i64, vp, vp, vp]
    L.mlora_probe_mfma8.argtypes = [i64, i64, vp, vp, vp]
    L.mlora_probe_copy.argtypes = [vp, vp, i64, vp]
    L.mlora_probe_read.argtypes = [vp, i64, vp, vp]
    L.mlora_probe_l2_to_lds.argtypes = [ctypes.c_int, i64, i64, vp, vp, vp]
    for f in (L.mlora_probe_mfma, L.mlora_probe_mfma8, L.mlora_probe_copy, L.mlora_probe_read,
              L.mlora_probe_l2_to_lds):
        f.restype = ctypes.c_int
    stream = vp(torch.cuda.current_stream().cuda_stream)

    def best(launch, reps=6):
        ts = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            rc = launch()
            b.record()
            if rc != 0:
                raise RuntimeError(f"probe launch failed: hipError {rc}")
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b))
        return min(ts[1:])                       # the first launch warms up

    out = {}
    n_wg, iters = 1024, 8192
    flops = n_wg * 4 * iters * 16 * 32768
    res = torch.empty(n_wg * 256, dtype=torch.float32, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(3)
    ops = {"random": torch.randn(4096, generator=g, device="cuda").to(torch.bfloat16),
           "zeros": torch.zeros(4096, dtype=torch.bfloat16, device="cuda")}
    for name, op in ops.items():
        if random_only and name != "random":
            continue
        ms = best(lambda: L.mlora_probe_mfma(n_wg, iters, vp(op.data_ptr()), vp(res.data_ptr()), stream))
        out[f"mfma_bf16_{name}_operands"] = {"achieved": flops / (ms * 1e-3) / 1e12, "unit": "TFLOP/s",
                                            "ms": ms}
    # MXFP8 instruction: E4M3 codes of random normal values (no NaN codes)
    op8 = torch.randn(8192, generator=g, device="cuda").to(torch.float8_e4m3fn).view(torch.uint8)
    ms = best(lambda: L.mlora_probe_mfma8(n_wg, iters // 2, vp(op8.data_ptr()), vp(res.data_ptr()), stream))
    out["mfma_mxfp8_random_operands"] = {"achieved": n_wg * 4 * (iters // 2) * 16 * 131072 / (ms * 1e-3) / 1e12,
                                         "unit": "TFLOP/s", "ms": ms}
    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    ms = best(lambda: L.mlora_probe_copy(vp(src.data_ptr()), vp(dst.data_ptr()), nbytes, stream))
    out["hbm_copy"] = {"achieved": 2 * nbytes / (ms * 1e-3) / 1e9, "unit": "GB/s", "ms": ms,
                       "bytes_per_launch": 2 * nbytes}
    red = torch.empty(2048 * 256, dtype=torch.float32, device="cuda")
    ms = best(lambda: L.mlora_probe_read(vp(src.data_ptr()), nbytes, vp(red.data_ptr()), stream))
    out["hbm_read"] = {"achieved": (nbytes + red.numel() * 4) / (ms * 1e-3) / 1e9, "unit": "GB/s", "ms": ms,
                       "bytes_per_launch": nbytes + red.numel() * 4}
    # operand blocks from L2 into LDS, one workgroup per CU, each on its own 64 KiB slab
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    l2l_iters = 2000
    l2l_out = torch.empty(ncu * 256, dtype=torch.int32, device="cuda")
    for path, name in ((0, "l2_to_lds_direct"), (1, "l2_to_lds_staged"), (2, "l2_to_registers")):
        ms = best(lambda: L.mlora_probe_l2_to_lds(path, ncu, l2l_iters, vp(src.data_ptr()),
                                                   vp(l2l_out.data_ptr()), stream))
        moved = ncu * l2l_iters * 65536
        out[name] = {"achieved": moved / (ms * 1e-3) / 1e9, "unit": "GB/s", "ms": ms,
                     "per_cu": moved / ncu / (ms * 1e-3) / 1e9}
    del src, dst
    torch.cuda.empty_cache()
    return out


def time_steps(step, steps, warmup):
    """Wall time per step (ms) of ``step(i)``, synchronized on both sides."""
    import torch
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


OPT_BYTES_PER_ELEM = 30    # read p, g, m, v (fp32); write p, m, v (fp32) and the bf16 copy


def optimizer_step(w, plan, layer, steps, warmup, seed, clip=None):
    """The per-adapter AdamW step over the layer's adapters (fp32 masters and
    moments, bf16 copies written back into the layer's A_i, B_i), with every
    adapter stepping: launch time from events on its stream, against the HBM
    roofline of its algorithmic bytes.  With ``clip``, every adapter clips its
    gradients to that norm first (two more launches, timed as grad_norm; they
    read every gradient once more: 4 bytes per element)."""
    import torch
    from adapter_lora_segments_amd import AdamW, adamw_hparams
    from workloads import optim
    opt = AdamW(layer)
    hps = [dict(h, start=0) for h in optim.hyperparameters(plan.info["n"] * plan.info["n_proj"], seed)]
    if clip is not None:
        hps = [dict(h, max_grad_norm=float(clip)) for h in hps]
    hp = adamw_hparams(optim.step_hparams(hps, 0))
    on = clip is not None
    for _ in range(warmup):
        opt.step(hp, clip_grads=on)
    torch.cuda.synchronize()
    plan.profile_enable(["adamw", "grad_norm"])
    plan.profile_read()
    for _ in range(steps):
        opt.step(hp, clip_grads=on)
    torch.cuda.synchronize()
    prof = plan.profile_read()
    tot_ms, n = prof["adamw"]
    gn_ms, gn_n = prof["grad_norm"]
    plan.profile_enable(False)
    avg = tot_ms / max(n, 1)
    elems = sum(int(r) * (plan.info["d_in"] + int(wd)) for r, wd in zip(plan.ranks, plan.pair_widths))
    gbs = OPT_BYTES_PER_ELEM * elems / (avg * 1e-3) / 1e9
    out = {"kernel": "k_adamw (per-adapter AdamW, bf16 copies)", "elements": elems,
           "bytes_per_launch": OPT_BYTES_PER_ELEM * elems, "avg_launch_ms": avg, "launches": n,
           "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": gbs / PEAK_HBM_GBS}}
    if on:
        gavg = gn_ms / max(gn_n, 1)
        ggbs = 4 * elems / (gavg * 1e-3) / 1e9
        out["clip"] = {"max_grad_norm": float(clip), "kernels": "k_grad_sq + k_clip_coef",
                       "bytes_per_launch": 4 * elems, "avg_launch_ms": gavg, "launches": gn_n,
                       "roofline": {"bound": "hbm", "achieved": ggbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                    "frac": ggbs / PEAK_HBM_GBS}}
    return out


def sequential_layers(w, q, d, sets, layout="kn", layer_w0=None):
    """The same work as one library call per adapter: a one-adapter plan per
    non-empty segment over its own rows (row slices of the packed tensors)."""
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    p = w.projections[q]
    off = [int(v) for v in d["offsets"]]
    out = []
    for i in range(w.n):
        lo, hi = off[i], off[i + 1]
        if hi == lo:
            continue
        plan = Plan([0, hi - lo], [int(d["ranks"][i])], p.d_in, p.d_out, "bf16", w0_layout=layout)
        W0 = layer_w0 if layer_w0 is not None else d["W0"]
        layer = PackedLoRALinear(plan, W0, [d["A"][i]], [d["B"][i]], [float(d["scales"][i])])
        Y = [torch.empty((hi - lo, p.d_out), dtype=torch.bfloat16, device="cuda") for _ in range(sets)]
        dX = [torch.empty((hi - lo, p.d_in), dtype=torch.bfloat16, device="cuda") for _ in range(sets)]
        out.append((lo, hi, plan, layer, Y, dX))
    return out


def packing_sweep(steps, warmup):
    """Packed against sequential over the shapes of the PLoRA page's Table 7
    (rank 64, hidden sizes 2048-18944 of two Qwen-2.5 models, 2 to 32
    adapters, batch 1): one plan over n adapters of 512 tokens each against
    n one-adapter calls, forward+backward of the whole layer (base GEMM
    included), synthetic bf16 data."""
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    g = torch.Generator(device="cuda").manual_seed(0)
    rows = []
    for d_in, d_out in ((2048, 2048), (3584, 3584), (2048, 11008), (3584, 18944)):
        W0 = (torch.randn((d_in, d_out), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        for n in (1, 2, 4, 8, 16, 32):
            r, tok = 64, 512
            T = n * tok
            X = torch.randn((T, d_in), generator=g, device="cuda").to(torch.bfloat16)
            dY = torch.randn((T, d_out), generator=g, device="cuda").to(torch.bfloat16)
            A = [(torch.randn((d_in, r), generator=g, device="cuda") * d_in ** -0.5).to(torch.bfloat16)
                 for _ in range(n)]
            B = [(torch.randn((r, d_out), generator=g, device="cuda") * 0.01).to(torch.bfloat16)
                 for _ in range(n)]
            sc = [16.0 / r] * n
            plan = Plan(list(range(0, T + 1, tok)), [r] * n, d_in, d_out, "bf16")
            layer = PackedLoRALinear(plan, W0, A, B, sc)
            Y = torch.empty((T, d_out), dtype=torch.bfloat16, device="cuda")
            dX = torch.empty((T, d_in), dtype=torch.bfloat16, device="cuda")

            def packed(i):
                layer.forward(X, Y)
                layer.backward(dY, X, dX)
            t_p = time_steps(packed, steps, warmup)
            seq = []
            for i in range(n):
                pl = Plan([0, tok], [r], d_in, d_out, "bf16")
                seq.append((i * tok, PackedLoRALinear(pl, W0, [A[i]], [B[i]], [sc[i]])))

            def sequential(i):
                for lo, lay in seq:
                    lay.forward(X[lo:lo + tok], Y[lo:lo + tok])
                    lay.backward(dY[lo:lo + tok], X[lo:lo + tok], dX[lo:lo + tok])
            t_s = time_steps(sequential, steps, warmup)
            rows.append({"d_in": d_in, "d_out": d_out, "adapters": n, "rank": r, "tokens_per_adapter": tok,
                         "packed_ms": t_p, "sequential_ms": t_s, "speedup": t_s / t_p})
            print(f"# {d_in}x{d_out} n={n}: packed {t_p:.3f} ms, sequential {t_s:.3f} ms, "
                  f"{t_s / t_p:.2f}x", file=sys.stderr, flush=True)
            del layer, plan, seq, X, dY, A, B, Y, dX
    return rows


def cost_table(steps, warmup):
    """Kernel cost table T(r, n, d): one adapter of rank r over n tokens on a
    d x d layer (bf16, forward + backward), the step time and each kernel
    kind's share from events on its stream.  The shape of what a planner of
    packed LoRA jobs consumes (the PLoRA page's cost model, §3.2; its Table 7
    sizes span d 2048-18944 and ranks 8-128)."""
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    g = torch.Generator(device="cuda").manual_seed(0)
    rows = []
    for d in (2048, 4096, 8192):
        W0 = (torch.randn((d, d), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
        for n in (512, 2048, 8192):
            X = torch.randn((n, d), generator=g, device="cuda").to(torch.bfloat16)
            dY = torch.randn((n, d), generator=g, device="cuda").to(torch.bfloat16)
            Y = torch.empty_like(dY)
            dX = torch.empty_like(X)
            for r in (8, 32, 128):
                A = (torch.randn((d, r), generator=g, device="cuda") * d ** -0.5).to(torch.bfloat16)
                B = (torch.randn((r, d), generator=g, device="cuda") * 0.01).to(torch.bfloat16)
                plan = Plan([0, n], [r], d, d, "bf16")
                layer = PackedLoRALinear(plan, W0, [A], [B], [16.0 / r])

                def one(i):
                    layer.forward(X, Y)
                    layer.backward(dY, X, dX)
                ms = time_steps(one, steps, warmup)
                plan.profile_enable(True)
                plan.profile_read()
                for i in range(steps):
                    one(i)
                torch.cuda.synchronize()
                per = {k: v[0] / steps for k, v in plan.profile_read().items() if v[1]}
                plan.profile_enable(False)
                rows.append({"d": d, "tokens": n, "rank": r, "ms_per_step": ms,
                             "kernels_ms": {k: round(v, 5) for k, v in per.items()}})
                print(f"# d={d} n={n} r={r}: {ms:.4f} ms", file=sys.stderr, flush=True)
                del layer, plan, A, B
    return rows


def vendor_gemm(w, steps, warmup):
    """The library's base GEMM launches beside torch.matmul (hipBLASLt) on the
    same base products of the workload's first projection, in both W0
    layouts: forward X.W0 and dX = dY.W0^T.  Ours: mean event time of one
    launch of the forward GEMM (base plus fused expand) and of the dX GEMM
    (base plus dZ.A^T; timed beside the concurrent weight-gradient kernels),
    each from calls of that direction alone.  TFLOP/s count the base product
    only, 2 T d_in d_out."""
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    from workloads.tensors import device_tensors
    p = w.projections[0]
    d = device_tensors(w, 0, sets=1)
    X, dY = d["X"][0], d["dY"][0]
    T = X.shape[0]
    flops = 2.0 * T * p.d_in * p.d_out

    def ev(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    out = {}
    Wkn = d["W0"]
    Wnk = Wkn.t().contiguous()
    Y = torch.empty((T, p.d_out), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((T, p.d_in), dtype=torch.bfloat16, device="cuda")
    for layout, W0 in (("kn", Wkn), ("nk", Wnk)):
        plan = Plan(d["offsets"], d["ranks"], p.d_in, p.d_out, "bf16", n_streams=1, w0_layout=layout)
        layer = PackedLoRALinear(plan, W0, d["A"], d["B"], d["scales"])
        layer.forward(X, Y)
        layer.backward(dY, X, dX)
        for kind, fn in (("gemm_fwd", lambda: layer.forward(X, Y)), ("gemm_dx", lambda: layer.backward(dY, X, dX))):
            plan.profile_enable([kind])
            plan.profile_read()
            ev(fn)
            ms, cnt = plan.profile_read()[kind]
            plan.profile_enable(False)
            ms /= max(cnt, 1)
            out[f"ours {kind} {layout}"] = {"us": ms * 1e3, "tflops": flops / (ms * 1e-3) / 1e12}
        del layer, plan
    for name, fn in (("torch fwd kn", lambda: torch.matmul(X, Wkn, out=Y)),
                     ("torch fwd nk", lambda: torch.matmul(X, Wnk.t(), out=Y)),
                     ("torch dx kn", lambda: torch.matmul(dY, Wkn.t(), out=dX)),
                     ("torch dx nk", lambda: torch.matmul(dY, Wnk, out=dX))):
        ms = ev(fn)
        out[name] = {"us": ms * 1e3, "tflops": flops / (ms * 1e-3) / 1e12}
    return {"shape": f"{T}x{p.d_in}x{p.d_out}", "results": out}


def _short_kernel_name(name):
    """A kernel's name without its argument list and return type; torch's
    elementwise kernels keep the functor that tells them apart."""
    n = name[5:] if name.startswith("void ") else name
    if "at::native" in n:
        for key in ("neg_kernel", "MulFunctor", "FillFunctor", "copy_kernel", "normal_kernel", "bfloat16_copy"):
            if key in n:
                return n.split("<")[0] + "<" + key + ">"
    depth, out = 0, []
    for ch in n:                    # cut at the first '(' outside template brackets
        if ch == "<":
            depth += 1
        elif ch == ">":
            depth -= 1
        elif ch == "(" and depth == 0:
            break
        out.append(ch)
    return "".join(out).strip()


def summarize_rocprof(root):
    """Per-(kernel, grid size) summary of the rocprofv3 CSV files under
    ``root``: dispatch count and average duration from kernel traces, and the
    average value of each counter from counter collections (FETCH_SIZE and
    WRITE_SIZE in KiB per dispatch)."""
    import csv
    import glob
    trace, ctr = {}, {}
    for path in sorted(glob.glob(os.path.join(root, "**", "*.csv"), recursive=True)):
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                name = row.get("Kernel_Name")
                if not name:
                    continue
                grid = row.get("Grid_Size") or row.get("Grid_Size_X") or "?"
                key = (_short_kernel_name(name), grid)
                if path.endswith("kernel_trace.csv"):
                    t = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
                    n, tot = trace.get(key, (0, 0.0))
                    trace[key] = (n + 1, tot + t)
                elif path.endswith("counter_collection.csv"):
                    c = row["Counter_Name"]
                    n, tot = ctr.setdefault(key, {}).get(c, (0, 0.0))
                    ctr[key][c] = (n + 1, tot + float(row["Counter_Value"]))
    lines = []
    if trace:
        lines.append(f"{'grid':>10s} {'calls':>6s} {'avg_us':>10s} {'total_ms':>10s}  kernel")
        for (k, g), (n, tot) in sorted(trace.items(), key=lambda kv: -kv[1][1]):
            lines.append(f"{g:>10s} {n:6d} {tot / n:10.1f} {tot / 1e3:10.2f}  {k}")
    if ctr:
        names = sorted({c for v in ctr.values() for c in v})
        lines.append(f"{'grid':>10s} {'calls':>6s} " + " ".join(f"{c + '/disp':>18s}" for c in names) + "  kernel")
        for (k, g), v in sorted(ctr.items()):
            n = max(v[c][0] for c in v)
            lines.append(f"{g:>10s} {n:6d} " +
                         " ".join(f"{v[c][1] / v[c][0]:18.1f}" if c in v else f"{'-':>18s}" for c in names) + f"  {k}")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="mlp70b_pair")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--streams", type=int, default=0)
    ap.add_argument("--nano-rows", type=int, default=0,
                    help="plan option: rows per nano-batch of the skinny products (0: the plan's default)")
    ap.add_argument("--chunk-per-rank", type=int, default=0,
                    help="plan option: reduction chunk rows per padded rank (0: the plan's default)")
    ap.add_argument("--chunk-max", type=int, default=0,
                    help="plan option: most rows in a reduction chunk (0: the plan's default)")
    ap.add_argument("--all-projections", action="store_true",
                    help="time every projection of the workload in each step (the default)")
    ap.add_argument("--first-projection", action="store_true",
                    help="time only the workload's first projection (tokens/s per layer is otherwise "
                         "T / the summed forward+backward time of every projection)")
    ap.add_argument("--summarize-rocprof", default=None, metavar="DIR",
                    help="only print a per-kernel summary of the rocprofv3 CSV output under DIR (no GPU)")
    ap.add_argument("--ceilings", action="store_true",
                    help="only measure this GPU's MFMA and HBM ceilings (libmlora_probes.so); one JSON line")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip measuring the MFMA and HBM ceilings beside the roofline")
    ap.add_argument("--no-one-group", action="store_true",
                    help="with several stream groups, skip timing the same layers planned as one group")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="first run one elementwise copy kernel (torch.neg on float32) reading and "
                         "writing this many MiB, to scale hardware byte counters")
    ap.add_argument("--no-profile", action="store_true",
                    help="do not bracket launches with events (for external profilers)")
    ap.add_argument("--no-sequential", action="store_true",
                    help="skip timing the same work as one library call per adapter (packed "
                         "against sequential, on the first timed projection)")
    ap.add_argument("--shuffled-ids", action="store_true",
                    help="rows in a shuffled caller order with one adapter id per token "
                         "(mlora_plan_from_ids) instead of contiguous segments")
    ap.add_argument("--no-optimizer", action="store_true",
                    help="skip timing the per-adapter AdamW step (mlora_adamw_step) of the first "
                         "timed projection")
    ap.add_argument("--fused", action="store_true",
                    help="time the whole layer with the projections that share an input fused into one "
                         "packed layer each (q/k/v, gate/up: mlora_plan_multi); implies --all-projections")
    ap.add_argument("--w0-format", default="bf16", choices=["bf16", "mxfp8", "mxfp4"],
                    help="store the frozen base in MXFP8 (E4M3 codes) or MXFP4 (E2M1 codes, two per byte), "
                         "with E8M0 scales per 32 inputs, decoded per call; implies --no-sequential")
    ap.add_argument("--act-format", default="bf16", choices=["bf16", "mxfp8"],
                    help="mxfp8: quantize the activations of the forward's base product to MXFP8 and run it "
                         "on the scaled matrix cores (needs --w0-format mxfp8 or mxfp4; the base is held as [d_out][d_in])")
    ap.add_argument("--w0-layout", default="kn", choices=["kn", "nk", "both"],
                    help="layout of the frozen base: [d_in][d_out], [d_out][d_in], or both (held once in "
                         "each layout, built before timing; the forward then reads [d_out][d_in])")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the same steps replayed from a captured HIP graph (one-group plans)")
    ap.add_argument("--clip", type=float, default=None,
                    help="the optimizer step clips each adapter's gradients to this 2-norm first")
    ap.add_argument("--optimizer-only", action="store_true",
                    help="run one forward+backward for real gradients, then time only the "
                         "per-adapter AdamW step of the first projection; one JSON line")
    ap.add_argument("--cost-table", action="store_true",
                    help="only measure the kernel cost table T(rank, tokens, hidden) of single-adapter "
                         "layers and print it as one JSON line")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="only time the base GEMM launches of the workload's first projection in both W0 "
                         "layouts beside torch.matmul (hipBLASLt) on the same products; one JSON line")
    ap.add_argument("--packing-sweep", action="store_true",
                    help="only run the packed-against-sequential sweep over Table 7's shapes and "
                         "print its results as one JSON line")
    a = ap.parse_args()
    if a.summarize_rocprof:
        print(summarize_rocprof(a.summarize_rocprof))
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only: the packed layer is measured on one device's "
              f"share (--gpus {a.gpus} requested)", file=sys.stderr)
        sys.exit(2)

    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear, device_check
    from workloads import load_workload
    from workloads.multi import LAYER_GROUPS, device_multi
    from workloads.mx import quantize_mx_device, quantize_mx4_device
    from workloads.tensors import device_tensors

    torch.cuda.set_device(0)
    device_check()
    if a.cost_table:
        steps = min(a.steps, 20)
        rows = cost_table(steps, min(a.warmup, 5))
        print(json.dumps({"metric": "single-adapter fwd+bwd time per layer T(rank, tokens, hidden)",
                          "unit": "ms", "steps": steps, "data": "synthetic", "dtype": "bf16",
                          "results": rows}), flush=True)
        return
    if a.ceilings:
        print(json.dumps({"metric": "measured ceilings of this GPU", "data": "synthetic",
                          "ceilings": ceilings()}), flush=True)
        return
    if a.packing_sweep:
        steps = min(a.steps, 20)
        rows = packing_sweep(steps, min(a.warmup, 5))
        print(json.dumps({"metric": "packed vs sequential fwd+bwd time per layer", "unit": "ms",
                          "steps": steps, "data": "synthetic", "results": rows}), flush=True)
        return
    w = load_workload(a.workload, a.seed)
    if w.dtype != "bf16":
        print(f"{w.name} is a {w.dtype} workload: the oracle-sized case of the parity tests; the bench "
              "times the bf16 workloads", file=sys.stderr)
        sys.exit(2)
    if a.vendor_gemm:
        steps = min(a.steps, 30)
        r = vendor_gemm(w, steps, min(a.warmup, 5))
        print(json.dumps({"metric": "base GEMM time per launch, library and torch.matmul", "unit": "us",
                          "workload": w.name, "steps": steps, "data": "synthetic", "dtype": "bf16", **r}),
              flush=True)
        return
    if a.fused:
        a.all_projections, a.no_sequential = True, True
    mx = a.w0_format in ("mxfp8", "mxfp4")
    if a.act_format == "mxfp8" and a.w0_format == "bf16":
        print("--act-format mxfp8 needs --w0-format mxfp8 or mxfp4", file=sys.stderr)
        sys.exit(2)
    mx_layout = "nk" if a.act_format == "mxfp8" else "kn"
    if mx:
        a.no_sequential = True
        if a.fused or a.shuffled_ids:
            print(f"--w0-format {a.w0_format} runs with segment plans of single projections", file=sys.stderr)
            sys.exit(2)
    projs = [0] if a.first_projection else list(range(len(w.projections)))
    SETS = 4
    layers = []
    groups = LAYER_GROUPS.get(w.name) if a.fused else None
    if a.fused and not groups:
        print(f"--fused: {w.name} has no projections that share an input", file=sys.stderr)
        sys.exit(2)
    # device inputs (drawn once) and output buffers, shared by every plan built over them
    datas = []
    for gname, gp in (groups or []):
        d = device_multi(w, gp, sets=SETS)
        D = sum(d["widths"])
        datas.append(("multi", d, [torch.empty((w.T, D), dtype=torch.bfloat16, device="cuda") for _ in range(SETS)],
                      [torch.empty((w.T, d["d_in"]), dtype=torch.bfloat16, device="cuda") for _ in range(SETS)]))
    for q in (projs if not groups else []):
        p = w.projections[q]
        d = device_tensors(w, q, sets=SETS)
        if mx:
            d["W0_codes"] = (quantize_mx4_device if a.w0_format == "mxfp4" else quantize_mx_device)(d["W0"], mx_layout)
            d["W0_bytes"] = d["W0_codes"].numel()
        datas.append(("single", d, [torch.empty((w.T, p.d_out), dtype=torch.bfloat16, device="cuda")
                                    for _ in range(SETS)],
                      [torch.empty((w.T, p.d_in), dtype=torch.bfloat16, device="cuda") for _ in range(SETS)]))

    chunk_opts = dict(chunk_per_rank=a.chunk_per_rank, chunk_max=a.chunk_max, nano_rows=a.nano_rows)

    def make_layers(n_streams):
        out = []
        for kind, d, Ys, dXs in datas:
            if kind == "multi":
                plan = Plan.multi(d["offsets"], d["ranks"], d["d_in"], d["widths"], "bf16", n_streams=n_streams,
                                  **chunk_opts)
                flat = lambda nested: [x for row in nested for x in row]
                layer = PackedLoRALinear(plan, d["W0"], flat(d["A"]), flat(d["B"]), flat(d["scales"]))
            else:
                if a.shuffled_ids:
                    ids = np.repeat(np.arange(w.n), np.diff(np.asarray(d["offsets"])))
                    ids = ids[np.random.default_rng(a.seed).permutation(w.T)]
                    plan = Plan.from_ids(ids, d["ranks"], d["d_in"], d["d_out"], "bf16", n_streams=n_streams,
                                         w0_layout=a.w0_layout, **chunk_opts)
                else:
                    plan = Plan(d["offsets"], d["ranks"], d["d_in"], d["d_out"], "bf16", n_streams=n_streams,
                                w0_format=a.w0_format, w0_layout=a.w0_layout if not mx else mx_layout,
                                act_format=a.act_format, **chunk_opts)
                if mx:
                    W0 = d["W0_codes"]
                elif a.w0_layout == "nk":
                    W0 = d.setdefault("W0_nk", d["W0"].t().contiguous())
                else:
                    W0 = d["W0"]
                layer = PackedLoRALinear(plan, W0, d["A"], d["B"], d["scales"])
            out.append((plan, layer, d, Ys, dXs))
        return out

    layers = make_layers(a.streams or w.n_streams)

    def step(i, lays=None):
        k = i % SETS
        for plan, layer, d, Ys, dXs in (lays if lays is not None else layers):
            layer.forward(d["X"][k], Ys[k])
            layer.backward(d["dY"][k], d["X"][k], dXs[k])

    def profile(kinds, lays):
        for plan, *_ in lays:
            plan.profile_enable(kinds)
            plan.profile_read()  # clear

    def collect(lays):
        tot = {}
        for plan, *_ in lays:
            for k, (ms, n) in plan.profile_read().items():
                m0, n0 = tot.get(k, (0.0, 0))
                tot[k] = (m0 + ms, n0 + n)
        return tot

    if a.calib_copy_mb:
        nel = a.calib_copy_mb * (1 << 20) // 4
        src = torch.ones(nel, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if a.optimizer_only:
        step(0)
        torch.cuda.synchronize()
        o = optimizer_step(w, layers[0][0], layers[0][1], a.steps, a.warmup, a.seed, a.clip)
        p0 = w.projections[0]
        print(json.dumps({"metric": "per-adapter AdamW step, bytes/s", "value": o["roofline"]["achieved"],
                          "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
                          "higher_is_better": True, "data": "synthetic", "dtype": "fp32",
                          "config": {"workload": f"{w.name}: {p0.name} {p0.d_in}x{p0.d_out}, "
                                                 f"{w.n} adapters, ranks {sorted(set(w.ranks))}"},
                          "optimizer": o}), flush=True)
        return
    for i in range(a.warmup):
        step(i)
    torch.cuda.synchronize()
    # Timed region: whole steps, with only the forward GEMM of the first
    # projection bracketed by events (its duration feeds the roofline); every
    # other launch runs back to back, as in training.
    prof = not a.no_profile
    for j, (plan, *_) in enumerate(layers):
        plan.profile_enable(["gemm_fwd"] if prof and j == 0 else False)
        plan.profile_read()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(i)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    gemm_rec = layers[0][0].profile_read()["gemm_fwd"] if prof else (0.0, 0)
    # The same layers planned as one stream group, timed the same way; with
    # several groups the forward-GEMM launches of different groups overlap on
    # their streams, so the roofline's per-launch time is taken here, where
    # each launch has the chip to itself.
    one_group = None
    ones = None
    if not a.no_one_group and any(pl.info["n_groups"] > 1 for pl, *_ in layers):
        ones = make_layers(1)
        for i in range(a.warmup):
            step(i, ones)
        for j, (plan, *_) in enumerate(ones):
            plan.profile_enable(["gemm_fwd"] if prof and j == 0 else False)
            plan.profile_read()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(a.steps):
            step(i, ones)
        torch.cuda.synchronize()
        el1 = time.perf_counter() - t0
        if prof:
            gemm_rec = ones[0][0].profile_read()["gemm_fwd"]
            ones[0][0].profile_enable(False)
        one_group = {"ms_per_step": el1 / a.steps * 1e3, "tokens_per_s": w.T * a.steps / el1,
                     "note": "the same layers, inputs and steps planned as one stream group"}

    # Per-kernel breakdown from a separate pass with every launch bracketed
    # (the events themselves lengthen that pass's steps; kernels that run
    # concurrently on two streams include each other's time), over the
    # one-group layers when the timed layers have several groups (whose
    # side-stream kernels overlap the GEMMs by design).
    kern = {}
    klayers = ones if ones is not None else layers
    if prof:
        nb = max(3, min(a.steps, 10))
        profile(True, klayers)
        for i in range(nb):
            step(i, klayers)
        torch.cuda.synchronize()
        kern = {k: (v[0] / nb * a.steps, v[1]) for k, v in collect(klayers).items()}
        # Isolated pass: a backward without dX runs the weight-gradient
        # kernels on the group's own stream, alone, for clean times.
        profile(True, klayers)
        for i in range(nb):
            k = i % SETS
            for plan, layer, d, Ys, dXs in klayers:
                layer.forward(d["X"][k], Ys[k])
                layer.backward(d["dY"][k], d["X"][k], want_dx=False)
        torch.cuda.synchronize()
        iso = {k: (v[0] / nb * a.steps, v[1]) for k, v in collect(klayers).items()}
        profile(False, klayers)

    del ones, klayers
    seq_ms = None
    if not a.no_sequential and not a.shuffled_ids:
        q0 = projs[0]
        d0 = layers[0][2]
        # the same base buffer and layout as the packed layer
        seq = sequential_layers(w, q0, d0, SETS, layers[0][0].w0_layout, layers[0][1].W0)

        def seq_step(i):
            k = i % SETS
            for lo, hi, plan, layer, Y, dX in seq:
                layer.forward(d0["X"][k][lo:hi], Y[k])
                layer.backward(d0["dY"][k][lo:hi], d0["X"][k][lo:hi], dX[k])
        seq_ms = time_steps(seq_step, min(a.steps, 50), min(a.warmup, 10))
        packed_ms = time_steps(lambda i: (layers[0][1].forward(d0["X"][i % SETS], layers[0][3][i % SETS]),
                                          layers[0][1].backward(d0["dY"][i % SETS], d0["X"][i % SETS],
                                                                layers[0][4][i % SETS])),
                               min(a.steps, 50), min(a.warmup, 10))

    # The same steps replayed from a HIP graph: one capture of a full
    # rotation of the input sets, replayed K / SETS times (plans with one
    # stream group; the library refuses capture of several).
    graph_ms = None
    if not a.no_graph and all(pl.info["n_groups"] == 1 for pl, *_ in layers):
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(SETS):
                step(i)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(SETS):
                step(i)
        reps = max(1, a.steps // SETS)
        for _ in range(max(1, a.warmup // SETS)):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) / (reps * SETS) * 1e3
        del graph

    opt_out = None
    if prof and not a.no_optimizer:
        opt_out = optimizer_step(w, layers[0][0], layers[0][1], a.steps, a.warmup, a.seed, a.clip)

    ms = el / a.steps * 1e3
    tok_s = w.T * a.steps / el
    F = sum(alg_flops(w, q) for q in projs)
    tflops = F / (ms * 1e-3) / 1e12
    p0 = w.projections[0]
    shapes = ", ".join(f"{w.projections[q].name} {w.projections[q].d_in}x{w.projections[q].d_out}"
                       for q in projs)
    if groups:
        shapes = "; ".join(f"{g} [" + ", ".join(f"{w.projections[q].name} {w.projections[q].d_in}x"
                                                f"{w.projections[q].d_out}" for q in gp) + "]"
                           for g, gp in groups)
        shapes = "fused groups sharing an input: " + shapes
    out = {
        "metric": "multi-LoRA fwd+bwd tokens/sec per layer",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": (f"{w.name}: {p0.d_in}x{p0.d_out} bf16, " if len(projs) == 1 else
                                f"{w.name}: projections {shapes}, bf16, ") +
                               f"{w.n} adapters, ranks {sorted(set(w.ranks))}, {w.T} tokens (seed {w.seed}), "
                               f"{layers[0][0].info['n_groups']} stream group(s)" +
                               (f"; one_group: the same planned as one stream group" if one_group else ""),
                   "T": w.T, "d_in": p0.d_in, "d_out": p0.d_out, "adapters": w.n,
                   "projections": [w.projections[q].name for q in projs],
                   "streams": layers[0][0].info["n_groups"],
                   "rows": "shuffled, per-token adapter ids" if a.shuffled_ids else "adapter segments",
                   "fused": [g for g, _ in groups] if groups else None,
                   "w0_format": a.w0_format, "w0_layout": a.w0_layout if not mx else mx_layout,
                   "act_format": a.act_format},
        "tflops": tflops,
        "pct_bf16_peak": 100.0 * tflops / PEAK_BF16_TFLOPS,
    }
    if kern:
        out["kernels_ms_per_step"] = {k: v[0] / a.steps for k, v in kern.items() if v[1]}
        units = [gp for _, gp in groups] if groups else [[q] for q in projs]
        out["kernel_rooflines"] = kernel_rooflines(w, units, kern, iso, a.steps, a.w0_format, a.act_format)
    if one_group is not None:
        out["one_group"] = one_group
    ceil = None if a.no_ceilings else ceilings()
    if ceil is not None:
        out["ceilings"] = ceil
    if prof:
        g_ms, g_n = gemm_rec
        if g_n:
            avg = g_ms / g_n
            per_step = g_n / a.steps      # launches of the first layer's forward GEMM per step
            first = groups[0][1] if groups else [0]
            ach = sum(gemm_fwd_flops(w, q) for q in first) / per_step / (avg * 1e-3) / 1e12
            kname = "+".join(w.projections[q].name for q in first)
            mxk = a.act_format == "mxfp8"
            peak = PEAK_FP8_TFLOPS if mxk else PEAK_BF16_TFLOPS
            out["roofline"] = {"kernel": (f"k_gemm_mx8 (MXFP8 base GEMM + fused bf16 expand) of {kname} " if mxk else
                                          f"k_gemm<fwd> (base GEMM + fused expand) of {kname} ") +
                                         f"{p0.d_in}x{sum(w.projections[q].d_out for q in first)}",
                               "bound": "mfma", "achieved": ach, "peak": peak,
                               "unit": "TFLOP/s", "frac": ach / peak,
                               "traffic": None if (groups or mx) else measured_traffic(w.name, a.w0_layout),
                               "avg_launch_ms": avg,
                               "timed_in": "one-group pass" if one_group is not None else "the timed steps"}
            if per_step > 1:
                out["roofline"]["note"] = "several group launches per step that overlap on their streams"
            if ceil is not None:
                mp = ceil["mfma_mxfp8_random_operands" if mxk else "mfma_bf16_random_operands"]["achieved"]
                out["roofline"]["measured_peak"] = mp
                out["roofline"]["frac_measured"] = ach / mp
    if seq_ms is not None:
        out["packed_vs_sequential"] = {
            "projection": w.projections[projs[0]].name, "packed_ms_per_step": packed_ms,
            "sequential_ms_per_step": seq_ms, "speedup": seq_ms / packed_ms,
            "sequential": f"{len(seq)} one-adapter library calls, each over its own rows"}
    if graph_ms is not None:
        out["graph_replay"] = {"ms_per_step": graph_ms, "tokens_per_s": w.T / (graph_ms * 1e-3),
                               "note": "the same steps replayed from one captured HIP graph"}
    if opt_out is not None:
        out["optimizer"] = opt_out
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, projs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
