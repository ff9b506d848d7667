"""Python binding of the C interface: argument marshalling only.

Names mirror include/mlora.h: ``mlora_plan`` builds a host plan,
``mlora_forward`` / ``mlora_backward`` launch the HIP kernels on torch
device tensors.  torch is used for device memory and the current stream;
every step of the layer runs in the library's kernels.
"""
from __future__ import annotations

import ctypes
from typing import Sequence

import numpy as np

from . import _lib
from ._lib import check, lib


def _torch():
    import torch  # imported first so libmlora binds to torch's HIP runtime
    return torch


class Plan:
    """Host plan for one packed layer (seg_offsets, ranks, d_in, d_out); through
    ``Plan.from_ids``, for rows in the caller's order with one adapter id per
    token; through ``Plan.multi``, for several projections sharing the input
    (ranks [n][n_proj], output widths per projection).

    ``ranks`` holds one rank per (adapter, projection) pair in the order
    i * n_proj + q, the order of the per-adapter pointer and scale arrays."""

    def __init__(self, seg_offsets, ranks, d_in: int, d_out: int, dtype: str = "bf16",
                 nano_rows: int = 0, n_streams: int = 0, chunk_min: int = 0, chunk_max: int = 0,
                 chunk_per_rank: int = 0, w0_layout: str = "kn", gemm_rows: int = 0, _ids=None,
                 _widths=None, w0_format: str = "bf16", act_format: str = "bf16", wg_overlap: str = "auto",
                 grad_accumulate: bool = False):
        rk = np.ascontiguousarray(np.asarray(ranks, dtype=np.int32))
        opts = _lib.PlanOpts(nano_rows, gemm_rows, n_streams, chunk_min, chunk_max, chunk_per_rank,
                             _lib.W0_LAYOUTS[w0_layout], _lib.W0_FORMATS[w0_format],
                             _lib.ACT_FORMATS[act_format], _lib.WG_OVERLAP[wg_overlap],
                             1 if grad_accumulate else 0)
        h = ctypes.c_void_p()
        widths = [int(d_out)] if _widths is None else [int(v) for v in _widths]
        if _widths is not None:
            P = len(widths)
            if rk.ndim != 2 or rk.shape[1] != P:
                raise ValueError("ranks must be [n][n_proj] for a multi-projection plan")
            n = int(rk.shape[0])
            rk = np.ascontiguousarray(rk.reshape(-1))
            w = np.ascontiguousarray(np.asarray(widths, dtype=np.int64))
            if _ids is not None:
                ids = np.ascontiguousarray(np.asarray(_ids, dtype=np.int32).reshape(-1))
                check(lib().mlora_plan_multi_from_ids(
                    n, int(ids.shape[0]), ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), P,
                    w.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                    rk.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(d_in), _lib.DTYPES[dtype],
                    ctypes.byref(opts), ctypes.byref(h)))
            else:
                off = np.ascontiguousarray(np.asarray(seg_offsets, dtype=np.int64))
                if off.shape != (n + 1,):
                    raise ValueError("seg_offsets must have n + 1 entries")
                check(lib().mlora_plan_multi(n, off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), P,
                                             w.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                             rk.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(d_in),
                                             _lib.DTYPES[dtype], ctypes.byref(opts), ctypes.byref(h)))
        elif _ids is None:
            n = int(rk.shape[0])
            off = np.ascontiguousarray(np.asarray(seg_offsets, dtype=np.int64))
            if off.shape != (n + 1,):
                raise ValueError("seg_offsets must have len(ranks) + 1 entries")
            check(lib().mlora_plan(n, off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                   rk.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(d_in),
                                   int(d_out), _lib.DTYPES[dtype], ctypes.byref(opts), ctypes.byref(h)))
        else:
            n = int(rk.shape[0])
            ids = np.ascontiguousarray(np.asarray(_ids, dtype=np.int32).reshape(-1))
            check(lib().mlora_plan_from_ids(n, int(ids.shape[0]),
                                            ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                            rk.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), int(d_in),
                                            int(d_out), _lib.DTYPES[dtype], ctypes.byref(opts),
                                            ctypes.byref(h)))
        self._L = lib()
        self._h = h
        inf = _lib.PlanInfo()
        check(lib().mlora_plan_get_info(h, ctypes.byref(inf)))
        self.info = {k: getattr(inf, k) for k, _ in _lib.PlanInfo._fields_}
        self.dtype = dtype
        self.w0_layout = w0_layout
        self.w0_format = w0_format
        self.act_format = act_format
        self.offsets = self.export("offsets") if _ids is not None else np.asarray(seg_offsets, dtype=np.int64)
        self.ranks = rk
        self.widths = widths
        self.n_proj = len(widths)
        # output width of each pair's B (the width of its projection)
        self.pair_widths = np.asarray([widths[v % len(widths)] for v in range(rk.shape[0])], dtype=np.int64)
        self._ws_uploaded = None

    @classmethod
    def from_ids(cls, token_adapter, ranks, d_in: int, d_out: int, dtype: str = "bf16", **opts):
        """mlora_plan_from_ids: token t belongs to adapter token_adapter[t]."""
        return cls(None, ranks, d_in, d_out, dtype, _ids=token_adapter, **opts)

    @classmethod
    def multi(cls, seg_offsets, ranks, d_in: int, widths, dtype: str = "bf16", **opts):
        """mlora_plan_multi: projections of output widths ``widths`` sharing
        the input; ranks [n][n_proj]."""
        return cls(seg_offsets, ranks, d_in, int(sum(widths)), dtype, _widths=widths, **opts)

    @classmethod
    def multi_from_ids(cls, token_adapter, ranks, d_in: int, widths, dtype: str = "bf16", **opts):
        """mlora_plan_multi_from_ids: projections sharing the input, rows in
        the caller's order with one adapter id per token."""
        return cls(None, ranks, d_in, int(sum(widths)), dtype, _widths=widths, _ids=token_adapter, **opts)

    @property
    def handle(self):
        return self._h

    def export(self, name: str) -> np.ndarray:
        tid = _lib.TABLES.index(name)
        nbytes = ctypes.c_size_t(0)
        check(lib().mlora_plan_export(self._h, tid, None, ctypes.byref(nbytes)))
        dt = np.int64 if name in _lib.TABLE_I64 else np.int32
        buf = np.zeros(nbytes.value // np.dtype(dt).itemsize, dtype=dt)
        check(lib().mlora_plan_export(self._h, tid, buf.ctypes.data_as(ctypes.c_void_p),
                                      ctypes.byref(nbytes)))
        if name in _lib.TABLE_COLS:
            buf = buf.reshape(-1, _lib.TABLE_COLS[name])
        return buf

    def __del__(self):
        # The library handle is held by the plan itself: at interpreter exit
        # the module globals lib() needs may already be gone.
        h = getattr(self, "_h", None)
        L = getattr(self, "_L", None)
        if h is not None and h.value and L is not None:
            L.mlora_plan_destroy(h)
            self._h = ctypes.c_void_p()

    # ---- device-side helpers (torch) ----
    def alloc_workspace(self, device="cuda"):
        torch = _torch()
        return torch.empty(max(1, self.info["workspace_bytes"]), dtype=torch.uint8, device=device)

    def alloc_z(self, device="cuda"):
        torch = _torch()
        dt = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        return torch.empty(max(1, self.info["z_elems"]), dtype=dt, device=device)

    def upload(self, ws, stream=None):
        torch = _torch()
        s = stream if stream is not None else torch.cuda.current_stream()
        check(lib().mlora_plan_upload(self._h, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                                      ctypes.c_void_p(s.cuda_stream)))
        self._ws_uploaded = ws

    def profile_enable(self, on=True):
        """True: time every kernel kind; False: none; or an iterable of kind
        names (``_lib.KERNELS``) to time only those."""
        if on is True:
            mask = -1
        elif not on:
            mask = 0
        else:
            mask = 0
            for k in on:
                mask |= 1 << _lib.KERNELS.index(k)
        check(lib().mlora_profile_enable(self._h, mask))

    def profile_read(self) -> dict:
        n = len(_lib.KERNELS)
        ms = (ctypes.c_double * n)()
        cnt = (ctypes.c_int64 * n)()
        check(lib().mlora_profile_read(self._h, ms, cnt))
        return {k: (ms[i], cnt[i]) for i, k in enumerate(_lib.KERNELS)}


def mlora_plan(seg_offsets, ranks, d_in, d_out, dtype="bf16", **opts) -> Plan:
    return Plan(seg_offsets, ranks, d_in, d_out, dtype, **opts)


def pointer_table(tensors: Sequence, device="cuda"):
    """Device int64 array of the data pointers of ``tensors``."""
    torch = _torch()
    return torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64, device=device)


def _p(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _check_t(t, name, shape, dtype, numel_min=None):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel_min is not None and t.numel() < numel_min:
        raise ValueError(f"{name} needs at least {numel_min} elements")


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _dt(plan):
    torch = _torch()
    return torch.bfloat16 if plan.dtype == "bf16" else torch.float32


def _npairs(plan):
    return plan.info["n"] * plan.info["n_proj"]


def _w0_shape(plan):
    i = plan.info
    if plan.w0_format == "mxfp8":  # element codes, then the block scale codes
        return (i["d_in"] * i["d_out"] + i["d_out"] * (i["d_in"] // 32),)
    if plan.w0_format == "mxfp4":  # element codes two to a byte, then the block scale codes
        return (i["d_in"] * i["d_out"] // 2 + i["d_out"] * (i["d_in"] // 32),)
    if plan.w0_layout == "both":   # [d_in][d_out], then its transpose
        return (2 * i["d_in"] * i["d_out"],)
    return (i["d_in"], i["d_out"]) if plan.w0_layout == "kn" else (i["d_out"], i["d_in"])


def mlora_base_transpose(W, out, stream=None):
    """out[c][r] = W[r][c] (bf16 or fp32, dimensions multiples of 64), by the
    library's transpose kernel."""
    torch = _torch()
    rows, cols = W.shape
    dt = _lib.DTYPES["bf16" if W.dtype == torch.bfloat16 else "fp32"]
    assert W.is_contiguous() and out.is_contiguous() and out.numel() == W.numel() and out.dtype == W.dtype
    check(lib().mlora_base_transpose(_p(W), _p(out), rows, cols, dt, _stream(stream)))
    return out


def base_both(W0_kn, stream=None):
    """The two-layout base buffer (MLORA_W0_BOTH) of a [d_in][d_out] weight:
    the weight, then its transpose [d_out][d_in] built by the library."""
    torch = _torch()
    d_in, d_out = W0_kn.shape
    buf = torch.empty(2 * d_in * d_out, dtype=W0_kn.dtype, device=W0_kn.device)
    buf[: d_in * d_out].view(d_in, d_out).copy_(W0_kn)
    mlora_base_transpose(W0_kn.contiguous(), buf[d_in * d_out:], stream)
    return buf


def _w0_dtype(plan):
    torch = _torch()
    return torch.uint8 if plan.w0_format in ("mxfp8", "mxfp4") else _dt(plan)


def mlora_forward(plan: Plan, X, W0, A_ptrs, B_ptrs, scales, Y, Z, ws, stream=None):
    """Y = X W0 + s_i (X A_i) B_i per segment; Z <- s_i X A_i (plan layout)."""
    torch = _torch()
    i = plan.info
    dt = _dt(plan)
    _check_t(X, "X", (i["T"], i["d_in"]), dt)
    _check_t(W0, "W0", _w0_shape(plan), _w0_dtype(plan))
    _check_t(Y, "Y", (i["T"], i["d_out"]), dt)
    _check_t(Z, "Z", None, dt, i["z_elems"])
    for nm, t in (("A_ptrs", A_ptrs), ("B_ptrs", B_ptrs)):
        _check_t(t, nm, (_npairs(plan),), torch.int64)
    _check_t(scales, "scales", (_npairs(plan),), torch.float32)
    check(lib().mlora_forward(plan.handle, _p(X), _p(W0), _p(A_ptrs), _p(B_ptrs), _p(scales),
                              _p(Y), _p(Z), _p(ws), ws.numel(), _stream(stream)))
    return Y, Z


def mlora_forward_noalloc(plan: Plan, X, W0, A_ptrs, B_ptrs, scales, Y, Z, stream=None):
    """mlora_forward with the library's static scratch instead of a
    workspace: nothing is allocated (layers whose buffers exceed the scratch
    are refused)."""
    torch = _torch()
    i = plan.info
    dt = _dt(plan)
    _check_t(X, "X", (i["T"], i["d_in"]), dt)
    _check_t(W0, "W0", _w0_shape(plan), _w0_dtype(plan))
    _check_t(Y, "Y", (i["T"], i["d_out"]), dt)
    _check_t(Z, "Z", None, dt, i["z_elems"])
    for nm, t in (("A_ptrs", A_ptrs), ("B_ptrs", B_ptrs)):
        _check_t(t, nm, (_npairs(plan),), torch.int64)
    _check_t(scales, "scales", (_npairs(plan),), torch.float32)
    check(lib().mlora_forward_noalloc(plan.handle, _p(X), _p(W0), _p(A_ptrs), _p(B_ptrs), _p(scales),
                                      _p(Y), _p(Z), _stream(stream)))
    return Y, Z


def mlora_backward(plan: Plan, dY, X, W0, A_ptrs, B_ptrs, scales, Z, dX, dA_ptrs, dB_ptrs, ws,
                   stream=None):
    """dX (optional) and fp32 dA_i, dB_i through the pointer tables."""
    torch = _torch()
    i = plan.info
    dt = _dt(plan)
    _check_t(dY, "dY", (i["T"], i["d_out"]), dt)
    _check_t(X, "X", (i["T"], i["d_in"]), dt)
    _check_t(W0, "W0", _w0_shape(plan), _w0_dtype(plan))
    _check_t(Z, "Z", None, dt, i["z_elems"])
    if dX is not None:
        _check_t(dX, "dX", (i["T"], i["d_in"]), dt)
    for nm, t in (("A_ptrs", A_ptrs), ("B_ptrs", B_ptrs), ("dA_ptrs", dA_ptrs), ("dB_ptrs", dB_ptrs)):
        _check_t(t, nm, (_npairs(plan),), torch.int64)
    _check_t(scales, "scales", (_npairs(plan),), torch.float32)
    check(lib().mlora_backward(plan.handle, _p(dY), _p(X), _p(W0), _p(A_ptrs), _p(B_ptrs),
                               _p(scales), _p(Z), _p(dX), _p(dA_ptrs), _p(dB_ptrs), _p(ws),
                               ws.numel(), _stream(stream)))
    return dX


def adamw_hparams(hparams: Sequence[dict], device="cuda"):
    """Device array of mlora_adamw_hparams from per-adapter mappings with
    lr, beta1, beta2, eps, weight_decay, step and optionally max_grad_norm."""
    torch = _torch()
    arr = (_lib.AdamwHparams * len(hparams))()
    for k, h in enumerate(hparams):
        arr[k] = _lib.AdamwHparams(h["lr"], h["beta1"], h["beta2"], h["eps"], h["weight_decay"],
                                   int(h["step"]), float(h.get("max_grad_norm", 0.0)))
    raw = np.frombuffer(bytes(arr), dtype=np.uint8).copy()
    return torch.from_numpy(raw).to(device)


def mlora_adamw_step(plan: Plan, hparams, A_ptrs, B_ptrs, dA_ptrs, dB_ptrs, mA_ptrs, vA_ptrs,
                     mB_ptrs, vB_ptrs, A_copy_ptrs, B_copy_ptrs, ws, stream=None, clip_grads=False):
    """One AdamW step of every adapter (fp32 masters and moments through the
    pointer tables; optional bf16 copies)."""
    torch = _torch()
    n = _npairs(plan)
    _check_t(hparams, "hparams", (n * ctypes.sizeof(_lib.AdamwHparams),), torch.uint8)
    for nm, t in (("A_ptrs", A_ptrs), ("B_ptrs", B_ptrs), ("dA_ptrs", dA_ptrs), ("dB_ptrs", dB_ptrs),
                  ("mA_ptrs", mA_ptrs), ("vA_ptrs", vA_ptrs), ("mB_ptrs", mB_ptrs), ("vB_ptrs", vB_ptrs)):
        _check_t(t, nm, (n,), torch.int64)
    for nm, t in (("A_copy_ptrs", A_copy_ptrs), ("B_copy_ptrs", B_copy_ptrs)):
        if t is not None:
            _check_t(t, nm, (n,), torch.int64)
    check(lib().mlora_adamw_step(plan.handle, _p(hparams), _p(A_ptrs), _p(B_ptrs), _p(dA_ptrs),
                                 _p(dB_ptrs), _p(mA_ptrs), _p(vA_ptrs), _p(mB_ptrs), _p(vB_ptrs),
                                 _p(A_copy_ptrs), _p(B_copy_ptrs), 1 if clip_grads else 0, _p(ws),
                                 ws.numel(), _stream(stream)))


def device_check() -> None:
    check(lib().mlora_device_check())


def _check_adapters(plan: Plan, A: Sequence, B: Sequence, scales) -> None:
    """The library reads A_i and B_i through raw device pointers with the
    plan's ranks and widths, so every tensor is checked here first: A_i is
    [d_in][r_i] and B_i is [r_i][w_i] (w_i its projection's width) in the
    plan's dtype, dense, on a GPU, 16-byte aligned."""
    n = _npairs(plan)
    if len(A) != n or len(B) != n:
        raise ValueError(f"expected {n} adapter tensors for A and for B, got {len(A)} and {len(B)}")
    if np.asarray(scales).size != n:
        raise ValueError(f"expected {n} scales, got {np.asarray(scales).size}")
    dt = _dt(plan)
    d_in = plan.info["d_in"]
    items = []
    for v in range(n):
        r, w = int(plan.ranks[v]), int(plan.pair_widths[v])
        items += [(f"A[{v}]", A[v], (d_in, r)), (f"B[{v}]", B[v], (r, w))]
    for name, t, shape in items:        # what the plan fixes, on every tensor first
        if t is None:
            raise ValueError(f"{name} is required")
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
        if t.dtype != dt:
            raise ValueError(f"{name} must be {dt}, got {t.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    for name, t, _ in items:            # then where the memory is
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.data_ptr() % 16 != 0:
            raise ValueError(f"{name} must be 16-byte aligned")


class PackedLoRALinear:
    """One packed layer with its adapters, buffers and pointer tables.

    Holds device tensors A_i, B_i (parameters), dA_i, dB_i (fp32 gradients),
    the saved activation Z and the workspace; ``forward``/``backward`` call the
    library.  Pointer tables are uploaded once at construction.
    """

    def __init__(self, plan: Plan, W0, A: Sequence, B: Sequence, scales, device="cuda"):
        torch = _torch()
        self.plan = plan
        both_2d = plan.w0_layout == "both" and W0 is not None and W0.dim() == 2
        if both_2d:
            want = (plan.info["d_in"], plan.info["d_out"])
            if tuple(W0.shape) != want:
                raise ValueError(f"a two-layout base is given as [d_in][d_out] = {want}, got {tuple(W0.shape)}")
        _check_adapters(plan, A, B, scales)
        if both_2d:
            W0 = base_both(W0)          # given as [d_in][d_out]: add its transpose once
        self.W0 = W0
        self.A = list(A)
        self.B = list(B)
        n = _npairs(plan)
        self.scales = torch.as_tensor(np.asarray(scales, dtype=np.float32).reshape(-1), device=device)
        self.dA = [torch.empty((plan.info["d_in"], int(r)), dtype=torch.float32, device=device)
                   for r in plan.ranks]
        self.dB = [torch.empty((int(r), int(w)), dtype=torch.float32, device=device)
                   for r, w in zip(plan.ranks, plan.pair_widths)]
        self.A_ptrs = pointer_table(self.A, device)
        self.B_ptrs = pointer_table(self.B, device)
        self.dA_ptrs = pointer_table(self.dA, device)
        self.dB_ptrs = pointer_table(self.dB, device)
        self.ws = plan.alloc_workspace(device)
        self.Z = plan.alloc_z(device)
        plan.upload(self.ws)

    def forward(self, X, Y=None, stream=None):
        torch = _torch()
        if Y is None:
            Y = torch.empty((self.plan.info["T"], self.plan.info["d_out"]), dtype=X.dtype, device=X.device)
        mlora_forward(self.plan, X, self.W0, self.A_ptrs, self.B_ptrs, self.scales, Y, self.Z,
                      self.ws, stream)
        return Y

    def backward(self, dY, X, dX=None, want_dx=True, stream=None):
        torch = _torch()
        if want_dx and dX is None:
            dX = torch.empty((self.plan.info["T"], self.plan.info["d_in"]), dtype=X.dtype, device=X.device)
        mlora_backward(self.plan, dY, X, self.W0, self.A_ptrs, self.B_ptrs, self.scales, self.Z,
                       dX if want_dx else None, self.dA_ptrs, self.dB_ptrs, self.ws, stream)
        return dX


class AdamW:
    """Per-adapter AdamW state of a PackedLoRALinear: fp32 master weights,
    first and second moments, and their pointer tables.

    For a bf16 layer the masters start as the fp32 values of the layer's bf16
    A_i and B_i, and every ``step`` writes the updated masters back into those
    bf16 tensors (rounded to nearest even), so the next forward uses them.
    For an fp32 layer the layer's own A_i and B_i are the masters.  Gradients
    are the layer's dA_i and dB_i as the last backward wrote them.
    """

    def __init__(self, layer: PackedLoRALinear, device="cuda"):
        torch = _torch()
        self.layer = layer
        bf16 = layer.plan.dtype == "bf16"
        self.A = [a.float().clone() for a in layer.A] if bf16 else layer.A
        self.B = [b.float().clone() for b in layer.B] if bf16 else layer.B
        self.mA = [torch.zeros_like(a) for a in self.A]
        self.vA = [torch.zeros_like(a) for a in self.A]
        self.mB = [torch.zeros_like(b) for b in self.B]
        self.vB = [torch.zeros_like(b) for b in self.B]
        tab = lambda ts: pointer_table(ts, device)
        self.A_ptrs, self.B_ptrs = tab(self.A), tab(self.B)
        self.mA_ptrs, self.vA_ptrs = tab(self.mA), tab(self.vA)
        self.mB_ptrs, self.vB_ptrs = tab(self.mB), tab(self.vB)
        self.copies = (layer.A_ptrs, layer.B_ptrs) if bf16 else (None, None)

    def step(self, hparams, stream=None, clip_grads=False):
        """hparams: per adapter a mapping (lr, beta1, beta2, eps,
        weight_decay, step, optionally max_grad_norm), or a device array
        from ``adamw_hparams``; clip_grads applies each adapter's
        max_grad_norm."""
        hp = hparams if hasattr(hparams, "data_ptr") else adamw_hparams(hparams, self.layer.ws.device)
        L = self.layer
        mlora_adamw_step(L.plan, hp, self.A_ptrs, self.B_ptrs, L.dA_ptrs, L.dB_ptrs, self.mA_ptrs,
                         self.vA_ptrs, self.mB_ptrs, self.vB_ptrs, self.copies[0], self.copies[1],
                         L.ws, stream, clip_grads)
        return hp
