"""Checks that pin the MXFP8 decoding oracle (oracle/mx.py) to facts other
than itself.

- every E4M3 code against torch.float8_e4m3fn (an independent decoder), and
  hand-worked codes of the format's definition: 1.0, 1.5, 2.0, the largest
  finite 448, the smallest normal 2^-6, the smallest subnormal 2^-9,
  negative zero, NaN;
- E8M0 scale codes: 127 is 1, 0 is 2^-127, 254 is 2^127, 255 is NaN;
- nearest-even rounding to bf16 on hand-worked bit patterns (ties both ways,
  a carry into the exponent, NaN kept);
- dequantization of both layouts: a block's scale covers exactly its 32
  consecutive inputs of one output column, and the two layouts give the same
  weight for transposed codes;
- torch float64 decoding and matmul of a small quantized layer against the
  oracle's decoded weight fed to the plain layer oracle.
MXFP4 (torch has no FP4 decoder, so these rest on the format's definition
worked by hand):
- all sixteen E2M1 codes: 0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives
  (code 8 is negative zero);
- the nibble order: the even element of a pair in the low four bits;
- dequantization of both layouts element by element against the hand
  table times the block's scale, and the two layouts against each other;
- 1.5 x 2^127 stays exact, 6 x 2^127 becomes bf16 infinity (anything from
  2^128 up overflows), a scale code of 255 is NaN;
- a small layer decoded with the hand table in torch float64 against the
  oracle's weight fed to the plain layer oracle.
Activations quantized to MXFP8 for the base product (the OCP conversion):
- blocks worked by hand: shared exponents from a block's largest magnitude
  (1.0 -> 2^-8; 2^100 -> 2^92; a bf16 subnormal clamped at 2^-127; zeros),
  element codes of exact values, both tie directions, a subnormal element,
  saturation at 448;
- element rounding against torch.float8_e4m3fn's conversion (nearest, ties
  to even) on scaled values below 448, and against the format's half-step
  error bound;
- the layer: activations already on the MXFP8 grid give exactly the plain
  oracle's Y; the adapters' term is computed on X itself (the layer minus
  its B = 0 form equals the plain oracle's LoRA term).
"""
from __future__ import annotations

import numpy as np

from oracle import lora as ol


def pin_e4m3_table_vs_torch(om):
    import torch
    codes = np.arange(256, dtype=np.uint8)
    t = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = om.decode_e4m3(codes)
    both_nan = np.isnan(t) & np.isnan(ours)
    assert np.array_equal(np.isnan(t), np.isnan(ours)), "NaN codes differ"
    assert np.array_equal(t[~both_nan], ours[~both_nan]), "E4M3 values differ from torch"
    assert np.array_equal(np.signbit(t[~both_nan]), np.signbit(ours[~both_nan])), "signed zero differs"


def pin_e4m3_hand_codes(om):
    want = {0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x7E: 448.0, 0x08: 2.0 ** -6, 0x01: 2.0 ** -9,
            0x07: 7 * 2.0 ** -9, 0x00: 0.0, 0xFE: -448.0, 0xB8: -1.0}
    got = om.decode_e4m3(np.asarray(list(want), dtype=np.uint8))
    assert np.array_equal(got, np.asarray(list(want.values()))), got
    assert np.signbit(om.decode_e4m3(np.asarray([0x80], dtype=np.uint8)))[0], "0x80 is negative zero"
    assert np.all(np.isnan(om.decode_e4m3(np.asarray([0x7F, 0xFF], dtype=np.uint8)))), "S.1111.111 is NaN"


def pin_e8m0(om):
    got = om.decode_e8m0(np.asarray([127, 0, 254, 128, 120], dtype=np.uint8))
    assert np.array_equal(got, [1.0, 2.0 ** -127, 2.0 ** 127, 2.0, 2.0 ** -7]), got
    assert np.isnan(om.decode_e8m0(np.asarray([255], dtype=np.uint8)))[0]


def pin_round_bf16(om):
    vals = [1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -7, -2.0, 2 - 2.0 ** -9, 0.0, 448.0 * 2.0 ** -9]
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC000, 0x4000, 0x0000, 0x3F60]
    got = om.round_bf16(np.asarray(vals))
    assert [int(x) for x in got] == want, [hex(int(x)) for x in got]
    n = om.round_bf16(np.asarray([np.nan]))[0]
    assert (int(n) & 0x7F80) == 0x7F80 and (int(n) & 0x7F) != 0, "NaN must stay NaN"


def pin_dequant_blocks_and_layouts(om):
    rng = np.random.default_rng(1)
    d_in, d_out = 96, 8
    codes = rng.integers(0, 0x7E, size=(d_in, d_out), dtype=np.uint8)   # KN, finite, non-negative
    scales = rng.integers(118, 130, size=(d_out, d_in // 32), dtype=np.uint8)
    w = ol.as_f64(om.dequant_w0(codes, scales, d_in, d_out, "kn"), "bf16")
    for n in range(d_out):
        for k in range(d_in):
            q = om.decode_e4m3(np.asarray([codes[k, n]], dtype=np.uint8))[0]
            assert w[k, n] == q * 2.0 ** (int(scales[n, k // 32]) - 127), (k, n)
    w_nk = ol.as_f64(om.dequant_w0(np.ascontiguousarray(codes.T), scales, d_in, d_out, "nk"), "bf16")
    assert np.array_equal(w, w_nk), "layouts disagree"


def pin_layer_vs_torch(om):
    import torch
    rng = np.random.default_rng(2)
    d_in, d_out, T = 64, 16, 5
    codes = rng.integers(0, 256, size=(d_in, d_out), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38                                   # no NaN codes
    scales = rng.integers(120, 128, size=(d_out, d_in // 32), dtype=np.uint8)
    X = rng.standard_normal((T, d_in))
    tq = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
    ts = torch.from_numpy(2.0 ** (scales.astype(np.float64) - 127)).T.repeat_interleave(32, dim=0)
    Yt = (torch.from_numpy(X) @ (tq * ts)).numpy()
    W = om.dequant_w0(codes, scales, d_in, d_out, "kn")
    A = [np.zeros((d_in, 1))]
    B = [np.zeros((1, d_out))]
    Y, _ = ol.forward(X, ol.as_f64(W, "bf16"), A, B, [1.0], [0, T], "fp32")
    assert np.allclose(Y, Yt, rtol=0, atol=1e-12 * max(1.0, np.abs(Yt).max())), "decoded layer differs from torch"


# E2M1 codes 0..15 by hand: S.EE.M, bias 1
E2M1_HAND = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def _pack4(codes):
    """[rows][cols] codes 0..15 -> [rows][cols/2] bytes, even element low."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def pin_e2m1_hand_table(om):
    got = om.decode_e2m1(np.arange(16, dtype=np.uint8))
    assert np.array_equal(got, np.asarray(E2M1_HAND)), got
    assert np.array_equal(np.signbit(got), np.arange(16) >= 8), "sign is bit 3"


def pin_e2m1_nibble_order(om):
    # byte 0x21: low nibble 1 (0.5) first, high nibble 2 (1.0) second; 0xF7: 6.0 then -6.0
    codes = om.unpack_e2m1(np.asarray([[0x21, 0xF7]], dtype=np.uint8), 1, 4)
    assert np.array_equal(om.decode_e2m1(codes)[0], [0.5, 1.0, 6.0, -6.0]), codes
    d_in, d_out = 32, 4
    w = om.dequant_w0(np.full((d_in, d_out // 2), 0x21, np.uint8), np.full((d_out, 1), 127, np.uint8),
                      d_in, d_out, "kn", fmt="mxfp4")
    assert np.array_equal(ol.as_f64(w, "bf16")[0], [0.5, 1.0, 0.5, 1.0]), "columns of a KN row pair up"


def pin_mxfp4_blocks_and_layouts(om):
    rng = np.random.default_rng(3)
    d_in, d_out = 96, 8
    codes = rng.integers(0, 16, size=(d_in, d_out), dtype=np.uint8)     # [k][n]
    scales = rng.integers(118, 132, size=(d_out, d_in // 32), dtype=np.uint8)
    w = ol.as_f64(om.dequant_w0(_pack4(codes), scales, d_in, d_out, "kn", fmt="mxfp4"), "bf16")
    for n in range(d_out):
        for k in range(d_in):
            assert w[k, n] == E2M1_HAND[codes[k, n]] * 2.0 ** (int(scales[n, k // 32]) - 127), (k, n)
    w_nk = ol.as_f64(om.dequant_w0(_pack4(codes.T), scales, d_in, d_out, "nk", fmt="mxfp4"), "bf16")
    assert np.array_equal(w, w_nk), "layouts disagree"


def pin_mxfp4_overflow_and_nan(om):
    d_in, d_out = 32, 2
    codes = np.zeros((d_in, d_out), dtype=np.uint8)
    codes[0] = [7, 15]                       # 6, -6
    codes[1] = [3, 1]                        # 1.5, 0.5
    w = om.dequant_w0(_pack4(codes), np.asarray([[254], [254]], np.uint8), d_in, d_out, "kn", fmt="mxfp4")
    assert int(w[0, 0]) == 0x7F80 and int(w[0, 1]) == 0xFF80, "6 x 2^127 is beyond bf16: infinity"
    assert int(w[1, 0]) == 0x7F40 and int(w[1, 1]) == 0x7E80, "1.5 x 2^127 and 0.5 x 2^127 are exact"
    wn = om.dequant_w0(_pack4(codes), np.asarray([[255], [127]], np.uint8), d_in, d_out, "kn", fmt="mxfp4")
    f = ol.as_f64(wn, "bf16")
    assert np.all(np.isnan(f[:, 0])) and not np.any(np.isnan(f[:, 1])), "scale 255 is NaN for its block only"


def pin_mxfp4_layer_vs_torch(om):
    import torch
    rng = np.random.default_rng(4)
    d_in, d_out, T = 64, 16, 5
    codes = rng.integers(0, 16, size=(d_in, d_out), dtype=np.uint8)
    scales = rng.integers(120, 128, size=(d_out, d_in // 32), dtype=np.uint8)
    X = rng.standard_normal((T, d_in))
    table = torch.tensor(E2M1_HAND, dtype=torch.float64)
    tq = table[torch.from_numpy(codes.astype(np.int64))]
    ts = torch.from_numpy(2.0 ** (scales.astype(np.float64) - 127)).T.repeat_interleave(32, dim=0)
    Yt = (torch.from_numpy(X) @ (tq * ts)).numpy()
    W = om.dequant_w0(_pack4(codes), scales, d_in, d_out, "kn", fmt="mxfp4")
    Y, _ = ol.forward(X, ol.as_f64(W, "bf16"), [np.zeros((d_in, 1))], [np.zeros((1, d_out))], [1.0], [0, T],
                      "fp32")
    assert np.allclose(Y, Yt, rtol=0, atol=1e-12 * max(1.0, np.abs(Yt).max())), "decoded layer differs from torch"


def _bits(vals):
    from workloads.tensors import f32_to_bf16_bits
    return f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def pin_act_quant_hand_blocks(om):
    # row 0: largest magnitude 1.0 -> shared exponent 0 - 8, scale code 119; elements x 2^8
    #   1.0 -> 256 = 1.000 x 2^8 -> 0x78; 0.30078125 -> 77 = 1.203 x 2^6 -> 9.625 eighths -> 10 -> 0x6A;
    #   -0.5 -> -128 -> 0xF0; 2^-16 -> 2^-8, subnormal 2 x 2^-9 -> 0x02; ties: 68 = 8.5 eighths x 2^3
    #   -> 8 -> 0x68, 76 = 9.5 eighths -> 10 -> 0x6A
    # row 1: 1.9921875 -> 510 and 1.75 -> 448 saturate to 0x7E; 1.5 -> 384 = 12 eighths x 2^5 -> 0x7C
    # row 2: zeros -> scale code 0, codes 0
    # row 3: largest 2^100 -> exponent 92, scale code 219; 2^100 -> 2^8 -> 0x78; 2^97 -> 2^5 -> 0x60
    # row 4: largest 2^-130 (a bf16 subnormal) -> 2^-138 clamped to 2^-127, code 0; 2^-130 -> 2^-3 -> 0x20
    x = np.zeros((5, 32), dtype=np.float32)
    x[0, :6] = [1.0, 0.30078125, -0.5, 2.0 ** -16, 0.265625, 0.296875]
    x[1, :3] = [1.9921875, 1.75, 1.5]
    x[3, :2] = [2.0 ** 100, 2.0 ** 97]
    x[4, 0] = 2.0 ** -130
    codes, sc = om.quantize_act_mxfp8(_bits(x))
    assert sc.shape == (5, 1) and sc[:, 0].tolist() == [119, 119, 0, 219, 0], sc[:, 0]
    assert codes[0, :7].tolist() == [0x78, 0x6A, 0xF0, 0x02, 0x68, 0x6A, 0x00], [hex(c) for c in codes[0, :7]]
    assert codes[1, :4].tolist() == [0x7E, 0x7E, 0x7C, 0x00]
    assert not codes[2].any()
    assert codes[3, :2].tolist() == [0x78, 0x60] and codes[4, 0] == 0x20
    # blocks are 32 inputs along the row: a second block gets its own scale
    y = np.zeros((1, 64), dtype=np.float32)
    y[0, 0], y[0, 32] = 1.0, 4.0
    codes, sc = om.quantize_act_mxfp8(_bits(y))
    assert sc[0].tolist() == [119, 121] and codes[0, 0] == 0x78 and codes[0, 32] == 0x78


def pin_act_quant_vs_torch_rounding(om):
    import torch
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((64, 256)) * np.exp2(rng.integers(-20, 20, size=(64, 1)))).astype(np.float32)
    X = _bits(x)
    codes, sc = om.quantize_act_mxfp8(X)
    from oracle.lora import as_f64
    v = as_f64(X, "bf16").reshape(64, 8, 32) / om.decode_e8m0(sc)[:, :, None]
    v = v.reshape(64, 256)
    ok = np.abs(v) < 448
    t = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(t[ok], codes[ok]), "element rounding differs from torch's E4M3 conversion"
    assert np.all(codes[~ok] & 0x7F == 0x7E)
    q = om.decode_e4m3(codes)
    normal = np.abs(v) >= 2.0 ** -6
    assert np.all(np.abs(q - v)[normal & ok] <= np.abs(v)[normal & ok] * 2.0 ** -4)
    assert np.all(np.abs(q - v)[~normal] <= 2.0 ** -10)
    # every block's largest magnitude lands in [256, 512) before saturation
    amax = np.abs(v).reshape(64, 8, 32).max(axis=2)
    assert np.all((amax >= 256) & (amax < 512))


def pin_forward_act_mx(om):
    from oracle import lora as ol
    rng = np.random.default_rng(8)
    d_in, d_out, ranks, toks = 64, 96, [3, 5], [7, 6]
    off = np.concatenate([[0], np.cumsum(toks)])
    T = int(off[-1])
    W0 = _bits(rng.standard_normal((d_in, d_out)) * 0.1)
    A = [_bits(rng.standard_normal((d_in, r)) * 0.2) for r in ranks]
    B = [_bits(rng.standard_normal((r, d_out)) * 0.2) for r in ranks]
    sc = np.asarray([0.5, -2.0], dtype=np.float32)
    # activations already on the MXFP8 grid (+-1, +-2, 0.5, 0 with every block's largest 2):
    # the quantizer is exact and the layer is the plain one
    grid = rng.choice([0.0, 1.0, -1.0, 2.0, -2.0, 0.5], size=(T, d_in))
    grid[:, ::32] = 2.0
    Xg = _bits(grid)
    Y, Z = om.forward_act_mx(Xg, W0, A, B, sc, off)
    Yp, Zp = ol.forward(Xg, W0, A, B, sc, off, "bf16")
    assert np.array_equal(Y, Yp), "activations on the MXFP8 grid must give the plain layer"
    # the adapters' term uses X itself: Y minus its B = 0 form is the plain oracle's LoRA term
    X = _bits(rng.standard_normal((T, d_in)))
    Y1, _ = om.forward_act_mx(X, W0, A, B, sc, off)
    Y0, _ = om.forward_act_mx(X, W0, A, [np.zeros_like(b) for b in B], sc, off)
    L1, _ = ol.forward(X, np.zeros_like(W0), A, B, sc, off, "bf16")
    assert np.allclose(Y1 - Y0, L1, rtol=1e-12, atol=1e-12)
    # and the base term uses the quantized X: it differs from X W0 by the quantization only
    Yb, _ = om.forward_act_mx(X, W0, A, [np.zeros_like(b) for b in B], sc, off)
    Xq = om.dequant_act(*om.quantize_act_mxfp8(X))
    assert np.allclose(Yb, Xq @ ol.as_f64(W0, "bf16"), rtol=1e-12, atol=1e-12)
    assert not np.allclose(Yb, ol.as_f64(X, "bf16") @ ol.as_f64(W0, "bf16"), rtol=1e-6)


ALL_PINS = [pin_e4m3_table_vs_torch, pin_e4m3_hand_codes, pin_e8m0, pin_round_bf16,
            pin_dequant_blocks_and_layouts, pin_layer_vs_torch, pin_e2m1_hand_table, pin_e2m1_nibble_order,
            pin_mxfp4_blocks_and_layouts, pin_mxfp4_overflow_and_nan, pin_mxfp4_layer_vs_torch,
            pin_act_quant_hand_blocks, pin_act_quant_vs_torch_rounding, pin_forward_act_mx]
