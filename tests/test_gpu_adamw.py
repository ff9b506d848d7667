"""Per-adapter AdamW step (mlora_adamw_step) on the GPU against the float64
oracle (oracle/adamw.py).

Seeded fp32 masters, gradients and per-adapter hyperparameters
(workloads/optim.py) go to both sides; each side carries its own state over
several steps.  Checked per adapter and tensor, at every step:
- m and v within the fp32 bar (1e-4, max-abs error over max-abs value);
- the weights within the fp32 bar of the accumulated update p_t - p_0, once
  the rounding of the stored fp32 weight is allowed for: each step rounds it
  twice (the decayed weight, then the updated one), at most 2^-24 |p| each,
  so |p_gpu - p| <= 1e-4 max|p_t - p_0| + 2 k 2^-24 |p| after k steps (with a
  learning rate of 5e-5 and |p| near 0.25 the rounding alone is about 3e-4
  of the update);
- adapters whose step number is <= 0 are untouched, bit for bit;
- the bf16 copies equal the GPU's own fp32 masters rounded to nearest even,
  bit for bit (the rounding decision is taken on the same fp32 value);
- with clipping on, every adapter's gradients are scaled by the oracle's clip
  factor (oracle.adamw.clip_coef over the adapter's whole A and B gradients
  in float64) before the update; the limits are set from each adapter's
  first-step gradient norm so that some adapters are clipped, some stay under
  their limit and some have clipping off.
Shapes: a small layer with ranks 1..256 (several pieces per tensor and
partial last pieces), an fp32 layer, the 4096x4096 layer of four adapters the
bench times (whole tensors), and the 8192x28672 projection of 32 adapters
(the largest layer of the workloads; sampled elements, every tensor's first
and last element included)."""
import numpy as np
import pytest

from oracle import adamw as oa
from tests.gpu_harness import TOL, say
from workloads import optim
from workloads.tensors import f32_to_bf16_bits

TOLF = TOL["fp32"]


def _layer(dt, ranks, d_in, d_out, seed, widths=None):
    """With ``widths`` the layer has projections sharing the input: ``ranks``
    then lists the (adapter, projection) pairs' ranks adapter-major, and pair
    v's B has widths[v % P] columns."""
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear, AdamW
    n = len(ranks)
    if widths is None:
        off = np.arange(n + 1, dtype=np.int64) * 3   # rows do not enter the optimizer step
        plan = Plan(off, ranks, d_in, d_out, dt)
        A32, B32 = optim.masters(ranks, d_in, d_out, seed)
    else:
        P = len(widths)
        off = np.arange(n // P + 1, dtype=np.int64) * 3
        plan = Plan.multi(off, np.asarray(ranks).reshape(-1, P), d_in, widths, dt)
        A32, B32 = [], []
        for v, r in enumerate(ranks):
            a, b = optim.masters([r], d_in, widths[v % P], seed * 100 + v)
            A32 += a
            B32 += b
    n = len(ranks)
    tdt = torch.bfloat16 if dt == "bf16" else torch.float32
    A = [torch.from_numpy(a).cuda().to(tdt) for a in A32]
    B = [torch.from_numpy(b).cuda().to(tdt) for b in B32]
    layer = PackedLoRALinear(plan, None, A, B, [1.0] * n)
    opt = AdamW(layer)
    for dst, src in zip(opt.A + opt.B, A32 + B32):
        dst.copy_(torch.from_numpy(src).cuda())
    torch.cuda.synchronize()
    return plan, layer, opt, A32, B32


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _err(got, want):
    den = float(np.max(np.abs(want))) if want.size else 0.0
    num = float(np.max(np.abs(got - want))) if want.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


CLIP_FACTORS = (0.3, 3.0, 0.0, 0.05)      # limit = factor x first-step norm; 0 turns clipping off


def _run(dt, ranks, d_in, d_out, n_steps, seed, sample=None, widths=None, clip=False):
    import torch
    plan, layer, opt, A32, B32 = _layer(dt, ranks, d_in, d_out, seed, widths)
    n = len(ranks)
    hps = optim.hyperparameters(n, seed)
    tensors = lambda i: [(opt.A[i], opt.mA[i], opt.vA[i], layer.A[i]),
                         (opt.B[i], opt.mB[i], opt.vB[i], layer.B[i])]
    # element indices checked per tensor (None: all)
    idx = {}
    rng = np.random.default_rng(seed + 1)
    for i in range(n):
        for k, p0 in enumerate((A32[i], B32[i])):
            if sample is None:
                idx[i, k] = None
            else:
                e = rng.choice(p0.size, min(sample, p0.size), replace=False)
                idx[i, k] = np.unique(np.concatenate([e, [0, p0.size - 1]]))
    take = lambda a, ik: a.reshape(-1) if idx[ik] is None else a.reshape(-1)[idx[ik]]

    def dev_take(t, ik):
        flat = t.reshape(-1)
        if idx[ik] is None:
            return flat
        return flat[torch.from_numpy(idx[ik]).cuda()]

    # oracle state: float64, sampled elements only when sampling
    p0 = {(i, k): take(a, (i, k)).astype(np.float64) for i in range(n) for k, a in enumerate((A32[i], B32[i]))}
    po = dict(p0)
    mo = {ik: np.zeros_like(v) for ik, v in p0.items()}
    vo = {ik: np.zeros_like(v) for ik, v in p0.items()}
    prev = None
    applied = {i: 0 for i in range(n)}
    worst = ("", 0.0)
    for s in range(n_steps):
        if widths is None:
            gA, gB = optim.gradients(ranks, d_in, d_out, seed, s)
        else:
            gA, gB = [], []
            for v, r in enumerate(ranks):
                a, b = optim.gradients([r], d_in, widths[v % len(widths)], seed * 100 + v, s)
                gA += a
                gB += b
        for i in range(n):
            layer.dA[i].copy_(torch.from_numpy(gA[i]).cuda())
            layer.dB[i].copy_(torch.from_numpy(gB[i]).cuda())
        hp = optim.step_hparams(hps, s)
        coef = [1.0] * n
        if clip:
            if s == 0:
                norms = [np.sqrt(np.sum(gA[i].astype(np.float64) ** 2) + np.sum(gB[i].astype(np.float64) ** 2))
                         for i in range(n)]
                limits = [float(np.float32(CLIP_FACTORS[i % len(CLIP_FACTORS)] * norms[i])) for i in range(n)]
            for i in range(n):
                hp[i]["max_grad_norm"] = limits[i]
                if hp[i]["step"] >= 1:
                    coef[i] = oa.clip_coef([gA[i], gB[i]], limits[i])
        plan.profile_enable(["adamw", "grad_norm"])
        plan.profile_read()
        opt.step(hp, clip_grads=clip)
        torch.cuda.synchronize()
        prof = plan.profile_read()
        assert prof["adamw"][1] == 1, "one optimizer launch per step"
        assert prof["grad_norm"][1] == (1 if clip else 0), "norms are taken only with clipping on"
        plan.profile_enable(False)
        state = {}
        for i in range(n):
            h = hp[i]
            applied[i] += h["step"] >= 1
            for k, g in enumerate((gA[i], gB[i])):
                ik = (i, k)
                p_d, m_d, v_d, c_d = tensors(i)[k]
                pg = dev_take(p_d, ik).double().cpu().numpy()
                mg = dev_take(m_d, ik).double().cpu().numpy()
                vg = dev_take(v_d, ik).double().cpu().numpy()
                state[ik] = (pg, mg, vg)
                po[ik], mo[ik], vo[ik] = oa.adamw_tensor(po[ik], take(g, ik) * coef[i], mo[ik], vo[ik], h["lr"],
                                                         h["beta1"], h["beta2"], h["eps"],
                                                         h["weight_decay"], h["step"])
                if h["step"] <= 0:
                    before = prev[ik] if prev is not None else (p0[ik], np.zeros_like(pg), np.zeros_like(pg))
                    for a, b, nm in zip((pg, mg, vg), before, "pmv"):
                        assert np.array_equal(a, b), f"step {s}: skipped adapter {i} changed {nm}"
                    continue
                rounding = 2 * applied[i] * 2.0 ** -24 * np.abs(po[ik])
                excess = np.maximum(np.abs(pg - po[ik]) - rounding, 0.0)
                upd = float(np.max(np.abs(po[ik] - p0[ik])))
                e_p = float(np.max(excess)) / upd if upd > 0 else (0.0 if not excess.any() else float("inf"))
                errs = {"p": e_p, "m": _err(mg, mo[ik]), "v": _err(vg, vo[ik])}
                for nm, e in errs.items():
                    if e > worst[1]:
                        worst = (f"step {s} adapter {i} {'AB'[k]} {nm}", e)
                    assert e <= TOLF, f"step {s} adapter {i} tensor {'AB'[k]}: {nm} err {e:.3e}"
                if dt == "bf16":
                    want = f32_to_bf16_bits(pg.astype(np.float32))
                    cb = _bits(c_d).reshape(-1)
                    got = cb if idx[ik] is None else cb[idx[ik]]
                    assert np.array_equal(got, want), f"step {s} adapter {i}: bf16 copy is not RNE of the master"
        prev = state
    say(f"  adamw {dt} ranks={list(ranks)[:8]}{'...' if len(ranks) > 8 else ''} {d_in}x{d_out} "
        f"{n_steps} steps{' clipped' if clip else ''}: worst {worst[0]} = {worst[1]:.3e} (tol {TOLF:.0e})")


@pytest.mark.gpu
@pytest.mark.parametrize("dt,ranks,d_in,d_out,steps", [
    ("bf16", [4, 16, 33, 64, 256, 8, 1], 256, 320, 4),
    ("fp32", [4, 8, 2, 100], 128, 192, 4),
])
def test_adamw_small_against_oracle(dt, ranks, d_in, d_out, steps):
    say(f"case adamw {dt} {ranks} {d_in}x{d_out}")
    _run(dt, ranks, d_in, d_out, steps, seed=3)


@pytest.mark.gpu
def test_adamw_bench_layer_whole():
    from workloads import load_workload
    w = load_workload("llama7b_proj", 0)
    p = w.projections[0]
    say(f"case adamw llama7b_proj {p.d_in}x{p.d_out} ranks {w.ranks}")
    _run("bf16", w.ranks, p.d_in, p.d_out, 3, seed=5)


@pytest.mark.gpu
def test_adamw_largest_layer_sampled():
    from workloads import load_workload
    w = load_workload("mlp70b_pair", 0)
    p = w.projections[0]
    say(f"case adamw mlp70b_pair {p.d_in}x{p.d_out}, {w.n} adapters (sampled)")
    _run("bf16", w.ranks, p.d_in, p.d_out, 2, seed=6, sample=512)


@pytest.mark.gpu
def test_adamw_projection_pairs():
    """A layer with projections sharing the input: every (adapter, projection)
    pair is its own optimizer unit, and B of a pair has its projection's width."""
    widths = [512, 256]
    ranks = [8, 64, 33, 1, 128, 16]          # three adapters x two projections, adapter-major
    say(f"case adamw projection pairs widths {widths} ranks {ranks}")
    _run("bf16", ranks, 256, None, 3, seed=8, widths=widths)


@pytest.mark.gpu
@pytest.mark.parametrize("dt,ranks,d_in,d_out,widths", [
    ("bf16", [4, 16, 33, 64, 256, 8, 1, 100], 256, 320, None),
    ("fp32", [4, 8, 2, 100], 128, 192, None),
    ("bf16", [8, 64, 33, 1, 128, 16, 4, 200], 256, None, [512, 256]),
])
def test_adamw_clipped_against_oracle(dt, ranks, d_in, d_out, widths):
    """Per-adapter gradient-norm clipping: clipped, unclipped and off adapters
    in one call, over steps where some adapters are skipped."""
    say(f"case adamw clipped {dt} ranks {ranks} {d_in}x{d_out} widths {widths}")
    _run(dt, ranks, d_in, d_out, 4, seed=9, widths=widths, clip=True)


@pytest.mark.gpu
def test_adamw_clipped_largest_layer_sampled():
    """Clipping over the 8192x28672 projection: each adapter's norm spans
    millions of elements (about a thousand work items per B)."""
    from workloads import load_workload
    w = load_workload("mlp70b_pair", 0)
    p = w.projections[0]
    say(f"case adamw clipped mlp70b_pair {p.d_in}x{p.d_out}, {w.n} adapters (sampled)")
    _run("bf16", w.ranks, p.d_in, p.d_out, 2, seed=10, sample=512, clip=True)
