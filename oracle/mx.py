"""Decoding of an MXFP8- or MXFP4-quantized frozen base weight, in float64
-- TEST INFRASTRUCTURE ONLY.

Parity pinned: see tests/pins_mx.py (the E4M3 code table against
torch.float8_e4m3fn and hand-worked codes of the format's definition; the
sixteen E2M1 codes and the nibble order worked by hand (torch cannot decode
FP4); the E8M0 scale codes; the nearest-even bf16 rounding against
hand-worked bit patterns, overflow included; and the dequantized layer
against torch float64 on the same codes).

What it follows: the PLoRA page (PLoRA: Efficient Concurrent LoRA Training
for Large Language Models, §5 and §11.3) trains adapters over a frozen base
that QLoRA-style methods keep in a low-precision format; only the adapters
are trained, so the base is read, never updated.  The format taken here is
the OCP microscaling format MXFP8 with E4M3 elements (the matrix cores of
the CDNA4 generation take it natively):
- an element code is S.EEEE.MMM with exponent bias 7: E = 0 gives the
  subnormal (-1)^S M 2^-9, 0 < E gives (-1)^S (8 + M) 2^(E - 10); the codes
  S.1111.111 are NaN; there is no infinity (largest finite 448);
- a block of 32 consecutive elements along the reduction dimension d_in
  shares one E8M0 scale code X: the scale is 2^(X - 127), and X = 255 is NaN;
- the weight the layer multiplies is the element times its block's scale,
  rounded to bf16 (nearest, ties to even).  For codes and scales whose
  products stay in bf16's normal range the product is exact (at most four
  significant bits), so the rounding only acts in the subnormal range.

The 4-bit base QLoRA uses (§11.3 of the page) is taken here as MXFP4, the
OCP microscaling format with E2M1 elements (the 4-bit format gfx950's matrix
cores take; QLoRA's own NF4 code book belongs to one library):
- an element code is S.EE.M with exponent bias 1: E = 0 gives the subnormal
  (-1)^S M / 2, 0 < E gives (-1)^S (2 + M) 2^(E - 2); the magnitudes are 0,
  0.5, 1, 1.5, 2, 3, 4 and 6; there is no NaN or infinity;
- two codes share a byte along the contiguous dimension of the layout, the
  even-indexed element in the low four bits;
- blocks, scales and the bf16 rounding are those of MXFP8.  Products of an
  element (at most two significant bits) and a scale are exact in bf16
  except above its range (2^128 and more, e.g. 2 x 2^127, become infinity)
  and deep in its subnormal range.

Activations for the base product on the scaled matrix cores.  With an MXFP8
base, the product X W0 can run on gfx950's MXFP8 x MXFP8 matrix
instructions; X is then quantized to MXFP8 as well, by the OCP
microscaling conversion, per row in blocks of 32 consecutive inputs (along
d_in, the reduction axis, as the base's blocks):
- the block's shared exponent is floor(log2(max |x|)) - 8 (8 being the
  largest exponent of an E4M3 element), clamped to [-127, 127]; a block of
  zeros takes -127; the E8M0 scale code is that exponent + 127;
- each element x / 2^exponent is rounded to the nearest E4M3 value, ties to
  even, and values from 448 up (the largest finite E4M3) saturate to 448.
The layer then computes Y = Q(X) W0 + s_i (X A_i) B_i: only the frozen
base's product uses the quantized activations; the adapters' shrink, the
saved Z' and the whole backward use X itself (the backward's dX through the
base is dY W0^T, the straight-through reading of the quantizer).

W0 codes are laid out like a bf16 W0 of the same layout (KN: [d_in][d_out],
NK: [d_out][d_in]), MXFP4 codes two to a byte along the row; scales are
[d_out][d_in / 32] in both layouts.
"""
from __future__ import annotations

import numpy as np


def decode_e4m3(codes) -> np.ndarray:
    """float64 values of E4M3 element codes (uint8)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    sub = m * 2.0 ** -9
    norm = (8 + m) * np.exp2(e - 10.0)
    v = s * np.where(e == 0, sub, norm)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def decode_e2m1(codes) -> np.ndarray:
    """float64 values of E2M1 element codes (the low four bits of each entry)."""
    c = np.asarray(codes).astype(np.int64) & 15
    s = np.where(c >> 3, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    return s * np.where(e == 0, 0.5 * m, (2 + m) * np.exp2(e - 2.0))


def unpack_e2m1(packed, rows, cols) -> np.ndarray:
    """The [rows][cols] element codes of bytes holding two each along a row,
    element 2j in the low four bits of byte j."""
    b = np.asarray(packed, dtype=np.uint8).reshape(rows, cols // 2)
    out = np.empty((rows, cols), dtype=np.uint8)
    out[:, 0::2] = b & 15
    out[:, 1::2] = b >> 4
    return out


def decode_e8m0(codes) -> np.ndarray:
    """float64 scales 2^(X - 127) of E8M0 codes; 255 is NaN."""
    x = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    return np.where(x == 255, np.nan, np.exp2(x - 127.0))


def round_bf16(v) -> np.ndarray:
    """Nearest-even bf16 of float64 values, returned as uint16 bit patterns.
    Exact for every value this module produces: the rounding is done on the
    value's float32 form, which holds a product of at most four significant
    bits and a power of two exactly unless it lies below float32's normal
    range, where float32 rounds first (such weights are far below any bf16
    weight that matters and are not produced by the workloads)."""
    with np.errstate(over="ignore"):          # beyond float32's range: infinity, as on the device
        f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    nan = np.isnan(f)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) & 0xFFFF
    r = np.where(nan, (u >> 16) | 0x40, r)
    return r.astype(np.uint16)


def dequant_w0(codes, scales, d_in, d_out, layout="kn", fmt="mxfp8"):
    """The bf16 weight the layer multiplies, as uint16 bit patterns in the
    math layout [d_in][d_out].  fmt: "mxfp8" (one E4M3 code per byte) or
    "mxfp4" (two E2M1 codes per byte)."""
    rows, cols = (d_in, d_out) if layout == "kn" else (d_out, d_in)
    if fmt == "mxfp4":
        q = decode_e2m1(unpack_e2m1(codes, rows, cols))
    else:
        q = decode_e4m3(codes).reshape(rows, cols)
    if layout != "kn":
        q = q.T
    sc = decode_e8m0(scales).reshape(d_out, d_in // 32)       # [n][k block]
    w = q * np.repeat(sc.T, 32, axis=0)                       # [d_in][d_out]
    return round_bf16(w)


def encode_e4m3(v) -> np.ndarray:
    """E4M3 codes (uint8) of float64 values, nearest with ties to even, from
    448 up saturating to 448 (finite inputs)."""
    v = np.asarray(v, dtype=np.float64)
    sign = np.signbit(v).astype(np.int64) << 7
    a = np.abs(v)
    code = np.zeros(a.shape, dtype=np.int64)
    sub = a < 2.0 ** -6                                  # subnormal range: steps of 2^-9
    code = np.where(sub, np.rint(a * 2.0 ** 9).astype(np.int64), code)   # 8 -> 0x08, the smallest normal
    _, ex = np.frexp(np.where(sub, 1.0, a))               # a = m 2^ex, m in [0.5, 1): floor(log2 a) = ex - 1
    e = ex - 1
    n = np.rint(np.where(sub, 8.0, a) * np.exp2(3.0 - e)).astype(np.int64)   # 8 .. 16: 1.mmm in eighths
    e = np.where(n == 16, e + 1, e)
    n = np.where(n == 16, 8, n)
    norm = ((e + 7) << 3) | (n - 8)
    code = np.where(sub, code, norm)
    code = np.where(a >= 448.0, 0x7E, code)
    return (sign | code).astype(np.uint8)


def quantize_act_mxfp8(X):
    """MXFP8 form of bf16 activations X ([T][K] uint16 bit patterns, K a
    multiple of 32): E4M3 element codes [T][K] and E8M0 scale codes
    [T][K / 32], by the conversion stated in this module's header."""
    from oracle.lora import as_f64
    x = as_f64(X, "bf16")
    T, K = x.shape
    blk = x.reshape(T, K // 32, 32)
    amax = np.max(np.abs(blk), axis=2)
    _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
    shared = np.where(amax > 0, np.clip(ex - 1 - 8, -127, 127), -127)
    v = blk / np.exp2(shared.astype(np.float64))[:, :, None]
    codes = encode_e4m3(v).reshape(T, K)
    return codes, (shared + 127).astype(np.uint8)


def dequant_act(codes, scales) -> np.ndarray:
    """float64 values of MXFP8 activations: element times its block's scale."""
    q = decode_e4m3(codes)
    T, K = q.shape
    return (q.reshape(T, K // 32, 32) * decode_e8m0(scales)[:, :, None]).reshape(T, K)


def forward_act_mx(X, W0, A, B, scales, offsets):
    """Y = Q(X) W0 + s_i (X_i A_i) B_i, float64, and the saved Z_i = X_i A_i:
    the base product over the MXFP8 form of the activations, the adapters
    over X itself.  X, W0 (the base as the layer multiplies it, e.g.
    dequant_w0's result), A_i, B_i are bf16 bit patterns."""
    from oracle.lora import as_f64
    Xq = dequant_act(*quantize_act_mxfp8(X))
    W = as_f64(W0, "bf16")
    o = [int(v) for v in offsets]
    Y = np.zeros((o[-1], W.shape[1]))
    Z = []
    for i in range(len(o) - 1):
        lo, hi = o[i], o[i + 1]
        Xi = as_f64(np.asarray(X)[lo:hi], "bf16")
        Zi = Xi @ as_f64(A[i], "bf16")
        Y[lo:hi] = Xq[lo:hi] @ W + float(scales[i]) * (Zi @ as_f64(B[i], "bf16"))
        Z.append(Zi)
    return Y, Z
