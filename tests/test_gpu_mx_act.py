"""MXFP8 activations on the scaled matrix cores (act_format = mxfp8, with an
MXFP8 or MXFP4 base held as [d_out][d_in]) on the GPU.

- The quantized activations the forward leaves in the workspace are
  bit-identical to the oracle's OCP conversion (oracle/mx.py,
  quantize_act_mxfp8), on rows made to hit its cases (a block of zeros,
  both tie directions, saturation at 448, a subnormal element, shared
  exponents clamped at 2^-127, a block of huge values) and on random rows.
- The layer against the oracle: Y against Q(X) W0 + s (X A) B, and Z', dZ,
  dX, dA, dB against the plain layer oracle over the decoded base (the
  backward is the straight-through one), within the bf16 bar; over
  segments, two stream groups and rows as shuffled per-token ids.
- Full size in the bench's configuration (the 4096x4096 layer, the
  8192x28672 projection of the 70B pair; with an MXFP4 base the 4096x4096
  layer and the 28672x8192 projection): Y on each adapter's first and last
  row plus 32 seeded rows.
Both bases are checked over segments, two stream groups and shuffled ids."""
import numpy as np
import pytest

from oracle import lora as ol
from oracle import mx as omx
from tests.gpu_harness import TOL, compare, custom_workload, say, to_dev, to_host_f64, workspace_dz
from workloads.mx import pack, quantize_mx, quantize_mx4
from workloads.tensors import f32_to_bf16_bits, host_tensors


def _act_region(plan, layer):
    """The MXFP8 activations of the last forward: codes [T][d_in], scales [T][d_in / 32]."""
    i = plan.info
    T, K = i["T"], i["d_in"]
    raw = layer.ws[i["act_offset"]:i["act_offset"] + T * K * 33 // 32].cpu().numpy()
    return raw[:T * K].reshape(T, K), raw[T * K:].reshape(T, K // 32)


def _mx_base(h, d_in, d_out, fmt="mxfp8"):
    q = quantize_mx4 if fmt == "mxfp4" else quantize_mx
    codes, sc = q(ol.as_f64(h["W0"], "bf16"), "nk")
    return codes, sc, omx.dequant_w0(codes, sc, d_in, d_out, "nk", fmt=fmt)


@pytest.mark.gpu
def test_activation_quantizer_bit_exact():
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    d_in, d_out = 256, 256
    w = custom_workload("mxact_q", "bf16", d_in, d_out, [8, 64], [40, 24], seed=6)
    h = host_tensors(w, 0)
    x = ol.as_f64(h["X"], "bf16").astype(np.float32)
    x[0, :6] = [1.0, 0.30078125, -0.5, 2.0 ** -16, 0.265625, 0.296875]     # ties, subnormal element
    x[0, 6:32] = 0.0
    x[1, 32:64] = 0.0
    x[1, 32:35] = [1.9921875, 1.75, -1.5]                                    # saturation
    x[2, 64:96] = 0.0                                                        # a block of zeros
    x[3, 0:32] = np.float32(2.0 ** 100) * np.sign(x[3, 0:32])                # huge block
    x[4, 0:32] = np.float32(2.0 ** -130)                                     # clamped exponent
    x[5] *= np.float32(2.0 ** -120)
    x[6] *= np.float32(2.0 ** 60)
    X = f32_to_bf16_bits(x)
    say("case mxfp8 activation quantizer: crafted and random rows")
    codes, sc, _ = _mx_base(h, d_in, d_out)
    plan = Plan(h["offsets"], h["ranks"], d_in, d_out, "bf16", w0_layout="nk", w0_format="mxfp8",
                act_format="mxfp8")
    layer = PackedLoRALinear(plan, torch.from_numpy(pack(codes, sc)).cuda(), [to_dev(a, "bf16") for a in h["A"]],
                             [to_dev(b, "bf16") for b in h["B"]], h["scales"])
    plan.profile_enable(["quant_act", "dequant"])
    plan.profile_read()
    layer.forward(to_dev(X, "bf16"))
    torch.cuda.synchronize()
    prof = plan.profile_read()
    assert prof["quant_act"][1] == 1 and prof["dequant"][1] == 0, "one quantizer launch, no decode of W0"
    got_c, got_s = _act_region(plan, layer)
    want_c, want_s = omx.quantize_act_mxfp8(X)
    assert np.array_equal(got_s, want_s), f"scales differ at {np.argwhere(got_s != want_s)[:5]}"
    bad = np.argwhere(got_c != want_c)
    assert bad.size == 0, f"codes differ at {bad[:5]}: {got_c[tuple(bad[0])]:#x} vs {want_c[tuple(bad[0])]:#x}"
    say(f"  {want_c.size} codes and {want_s.size} scales bit-identical")


CASES = [
    ("segments", 256, 384, [8, 64, 3, 200], [150, 300, 0, 77], 1, False),
    ("two groups", 512, 768, [16, 256, 33], [500, 9, 260], 2, False),
    ("ids", 384, 256, [32, 5, 128], [90, 260, 33], 1, True),
]


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("name,d_in,d_out,ranks,tokens,streams,ids", CASES)
def test_mxfp8_activation_layer_vs_oracle(name, d_in, d_out, ranks, tokens, streams, ids, fmt):
    """MXFP8 activations against an MXFP8 base (E4M3 x E4M3) or an MXFP4
    base (E2M1 first operand) on the scaled matrix instruction."""
    import torch
    from types import SimpleNamespace
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    say(f"case mxfp8 activations, {fmt} base, {name}: {d_in}x{d_out} ranks {ranks} tokens {tokens} "
        f"streams {streams}")
    w = custom_workload("mxact", "bf16", d_in, d_out, ranks, tokens, seed=9)
    h = host_tensors(w, 0)
    codes, sc, Wdec = _mx_base(h, d_in, d_out, fmt)
    off = h["offsets"]
    T = int(off[-1])
    opts = dict(n_streams=streams, w0_layout="nk", w0_format=fmt, act_format="mxfp8")
    if ids:
        tok = np.repeat(np.arange(len(ranks)), tokens)
        perm = np.random.default_rng(2).permutation(T)
        plan = Plan.from_ids(tok[perm], h["ranks"], d_in, d_out, "bf16", **opts)
        Xd, dYd = h["X"][perm], h["dY"][perm]
    else:
        plan = Plan(off, h["ranks"], d_in, d_out, "bf16", **opts)
        Xd, dYd = h["X"], h["dY"]
    layer = PackedLoRALinear(plan, torch.from_numpy(pack(codes, sc)).cuda(), [to_dev(a, "bf16") for a in h["A"]],
                             [to_dev(b, "bf16") for b in h["B"]], h["scales"])
    Y = layer.forward(to_dev(Xd, "bf16"))
    dX = layer.backward(to_dev(dYd, "bf16"), to_dev(Xd, "bf16"))
    torch.cuda.synchronize()
    Yh, dXh = to_host_f64(Y), to_host_f64(dX)
    got_c, got_s = _act_region(plan, layer)
    want_c, want_s = omx.quantize_act_mxfp8(Xd)              # the caller's row order, as the device holds it
    assert np.array_equal(got_c, want_c) and np.array_equal(got_s, want_s), "quantized activations differ"
    X, dY = Xd, dYd
    if ids:                                                  # the oracle takes rows grouped as the plan groups them
        G = plan.export("perm")
        X, dY, Yh, dXh = Xd[G], dYd[G], Yh[G], dXh[G]
    out = {"Y": Yh, "dX": dXh, "dA": [to_host_f64(t) for t in layer.dA], "dB": [to_host_f64(t) for t in layer.dB],
           "Z": to_host_f64(layer.Z), "dZ": workspace_dz(plan, layer), "plan": plan}
    hh = dict(h, X=X, dY=dY, W0=Wdec)
    # the backward, Z' and dZ against the plain oracle over the decoded base; Y is checked below
    errs = compare(SimpleNamespace(dtype="bf16"), hh, dict(out, Y=ol.forward(X, Wdec, h["A"], h["B"], h["scales"],
                                                                                  off, "bf16")[0]),
                   what=f"mxfp8 activations, {fmt} base, {name} (backward)")
    Yo, _ = omx.forward_act_mx(X, Wdec, h["A"], h["B"], h["scales"], off)
    e = ol.max_rel_err(Yh, Yo)
    # and the quantization is visible: Y differs from the bf16-activation layer's
    Yp, _ = ol.forward(X, Wdec, h["A"], h["B"], h["scales"], off, "bf16")
    say(f"  Y against Q(X) W0 + s (X A) B: {e:.3e}; against X W0 + ...: {ol.max_rel_err(Yh, Yp):.3e}")
    assert e <= TOL["bf16"] and e < ol.max_rel_err(Yh, Yp)


@pytest.mark.gpu
@pytest.mark.parametrize("workload,proj,fmt", [("llama7b_proj", 0, "mxfp8"), ("mlp70b_pair", 0, "mxfp8"),
                                               ("llama7b_proj", 0, "mxfp4"), ("mlp70b_pair", 1, "mxfp4")])
def test_mxfp8_activations_full_size(workload, proj, fmt):
    import torch
    from adapter_lora_segments_amd import Plan, PackedLoRALinear
    from tests.test_gpu_fullsize import stratified_rows
    from workloads import load_workload
    from workloads.mx import quantize_mx_device, quantize_mx4_device
    from workloads.tensors import device_tensors
    w = load_workload(workload, 0)
    p = w.projections[proj]
    say(f"case mxfp8 activations, {fmt} base, full size {workload}/{p.name} ({p.d_in}x{p.d_out}, T={w.T})")
    d = device_tensors(w, proj)
    q = quantize_mx4_device if fmt == "mxfp4" else quantize_mx_device
    Wmx = q(d["W0"], "nk")                                           # [d_out][d_in] codes, then scales
    plan = Plan(d["offsets"], d["ranks"], p.d_in, p.d_out, "bf16", n_streams=w.n_streams, w0_layout="nk",
                w0_format=fmt, act_format="mxfp8")
    layer = PackedLoRALinear(plan, Wmx, d["A"], d["B"], d["scales"])
    X = d["X"][0]
    Y = layer.forward(X)
    torch.cuda.synchronize()
    rows = stratified_rows(d["offsets"], np.random.default_rng(3))
    rt = torch.from_numpy(rows).cuda()
    gY = Y.index_select(0, rt).float().cpu().numpy()
    bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    Xr = bits(X.index_select(0, rt))
    raw = Wmx.cpu().numpy()
    ncb = p.d_in * p.d_out // (2 if fmt == "mxfp4" else 1)          # code bytes
    codes = raw[:ncb].reshape(p.d_out, -1)
    sc = raw[ncb:].reshape(p.d_out, p.d_in // 32)
    Wdec = omx.dequant_w0(codes, sc, p.d_in, p.d_out, "nk", fmt=fmt)
    own = ol.adapter_of_rows(d["offsets"], rows)
    sub_off = np.concatenate([[0], np.cumsum(np.bincount(own, minlength=w.n))])
    Yo, _ = omx.forward_act_mx(Xr, Wdec, [bits(a) for a in d["A"]], [bits(b) for b in d["B"]], d["scales"], sub_off)
    e = ol.max_rel_err(gY, Yo)
    say(f"  {len(rows)} rows: Y against Q(X) W0 + s (X A) B {e:.3e}")
    assert e <= TOL["bf16"]
