"""Seeded MXFP8 and MXFP4 base weights: a float weight quantized to E4M3
(or E2M1) element codes with one E8M0 scale per 32 consecutive inputs of an
output column.

MXFP4: per block the scale exponent is ceil(log2(amax / 6)) (6 is E2M1's
largest value), and each element w / 2^E takes the nearest of the eight
E2M1 magnitudes (ties to the smaller one) and the sign of w; two codes go to
a byte along the layout's rows, the even element in the low four bits.

The quantizer only makes inputs: per block the scale exponent is
ceil(log2(amax / 448)) (448 is E4M3's largest finite value), and the
elements are w / 2^E cast to E4M3 by torch (nearest even).  The layer only
ever decodes; no decoding lives here.  Codes are laid out like the bf16 W0
of the same layout, scales as [d_out][d_in / 32]; ``pack`` concatenates the
two into the buffer the library takes.
"""
from __future__ import annotations

import numpy as np


def quantize_mx(w, layout="kn"):
    """w: float array [d_in][d_out] (math layout).  Returns (codes uint8 in
    the given layout, scales uint8 [d_out][d_in / 32])."""
    import torch
    w = torch.as_tensor(np.asarray(w, dtype=np.float32))
    d_in, d_out = w.shape
    blocks = w.reshape(d_in // 32, 32, d_out)
    amax = blocks.abs().amax(dim=1)                                          # [d_in/32][d_out]
    e = torch.ceil(torch.log2(torch.clamp(amax, min=2.0 ** -120) / 448.0))
    x = torch.clamp(e + 127, 0, 254)
    q = blocks / torch.exp2(x - 127).unsqueeze(1)
    codes = q.reshape(d_in, d_out).to(torch.float8_e4m3fn).view(torch.uint8)
    if layout != "kn":
        codes = codes.T.contiguous()
    scales = x.to(torch.uint8).T.contiguous()
    return codes.numpy(), scales.numpy()


def quantize_mx_device(w_bf16, layout="kn"):
    """The same on the device from a torch bf16 [d_in][d_out] tensor; returns
    the packed uint8 buffer (codes, then scales)."""
    import torch
    w = w_bf16.float()
    d_in, d_out = w.shape
    blocks = w.reshape(d_in // 32, 32, d_out)
    amax = blocks.abs().amax(dim=1)
    e = torch.ceil(torch.log2(torch.clamp(amax, min=2.0 ** -120) / 448.0))
    x = torch.clamp(e + 127, 0, 254)
    q = (blocks / torch.exp2(x - 127).unsqueeze(1)).reshape(d_in, d_out)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8)
    if layout != "kn":
        codes = codes.T.contiguous()
    scales = x.to(torch.uint8).T.contiguous()
    return torch.cat([codes.reshape(-1), scales.reshape(-1)])


def pack(codes, scales):
    return np.concatenate([np.ascontiguousarray(codes).reshape(-1), np.ascontiguousarray(scales).reshape(-1)])


E2M1_MAGNITUDES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)


def _mx4_codes(q):
    """float32 torch tensor of scaled elements -> uint8 E2M1 codes (one per
    element, in the low four bits)."""
    import torch
    mags = torch.tensor(E2M1_MAGNITUDES, dtype=q.dtype, device=q.device)
    idx = torch.argmin((q.abs().unsqueeze(-1) - mags).abs(), dim=-1)        # first minimum: ties go low
    return (idx | ((q < 0).to(idx.dtype) << 3)).to(torch.uint8)


def _pack_pairs(c):
    return (c[:, 0::2] | (c[:, 1::2] << 4)).contiguous()


def _quantize_mx4(w, layout):
    import torch
    d_in, d_out = w.shape
    blocks = w.reshape(d_in // 32, 32, d_out)
    amax = blocks.abs().amax(dim=1)
    e = torch.ceil(torch.log2(torch.clamp(amax, min=2.0 ** -120) / 6.0))
    x = torch.clamp(e + 127, 0, 254)
    q = (blocks / torch.exp2(x - 127).unsqueeze(1)).reshape(d_in, d_out)
    c = _mx4_codes(q)
    if layout != "kn":
        c = c.T.contiguous()
    return _pack_pairs(c), x.to(torch.uint8).T.contiguous()


def quantize_mx4(w, layout="kn"):
    """w: float array [d_in][d_out] (math layout).  Returns (packed codes
    uint8 [rows][cols / 2] of the given layout, scales uint8 [d_out][d_in / 32])."""
    import torch
    codes, scales = _quantize_mx4(torch.as_tensor(np.asarray(w, dtype=np.float32)), layout)
    return codes.numpy(), scales.numpy()


def quantize_mx4_device(w_bf16, layout="kn"):
    """The same on the device from a torch bf16 [d_in][d_out] tensor; returns
    the packed uint8 buffer (codes, then scales)."""
    import torch
    codes, scales = _quantize_mx4(w_bf16.float(), layout)
    return torch.cat([codes.reshape(-1), scales.reshape(-1)])


def pack_e2m1(codes):
    """[rows][cols] E2M1 codes (0..15) -> [rows][cols / 2] bytes, the even
    element of each pair in the low four bits."""
    c = np.asarray(codes, dtype=np.uint8)
    return np.ascontiguousarray(c[:, 0::2] | (c[:, 1::2] << 4))
