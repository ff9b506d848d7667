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
