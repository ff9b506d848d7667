"""ctypes declarations of libmlora.so (include/mlora.h)."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmlora.so")

MLORA_OK = 0
STATUS = {0: "MLORA_OK", -1: "MLORA_ERR_INVALID_ARG", -2: "MLORA_ERR_UNSUPPORTED",
          -3: "MLORA_ERR_HIP", -4: "MLORA_ERR_WORKSPACE", -5: "MLORA_ERR_NOMEM"}
DTYPES = {"fp32": 0, "bf16": 1}
W0_LAYOUTS = {"kn": 0, "nk": 1, "both": 2}
W0_FORMATS = {"bf16": 0, "mxfp8": 1, "mxfp4": 2}
ACT_FORMATS = {"bf16": 0, "mxfp8": 1}
WG_OVERLAP = {"auto": 0, "side": 1, "after": 2}

TABLES = ["rpad", "zoff", "roff", "group_first_adapter", "nb", "nb_start", "chunks", "chunk_start",
          "chunk_rpref", "adapter_chunk_first", "adapter_chunk_count", "tiles", "tile_start", "ext",
          "tile_ext_start", "offsets", "ranks", "perm", "opt_blocks", "proj_cols", "seg_start",
          "chunk_boff", "ksplit", "opt_first"]
TABLE_COLS = {"nb": 3, "chunks": 3, "tiles": 2, "ext": 4, "opt_blocks": 2, "ksplit": 2}
TABLE_I64 = {"zoff", "offsets", "seg_start", "chunk_boff"}

KERNELS = ["shrink", "gemm_fwd", "dz", "token_reduce", "reduce", "gemm_dx", "prep", "adamw", "dequant",
           "grad_norm", "quant_act"]

# every symbol include/mlora.h declares
EXPORTS = ["mlora_plan", "mlora_plan_from_ids", "mlora_plan_multi", "mlora_plan_multi_from_ids", "mlora_plan_destroy", "mlora_plan_get_info", "mlora_plan_export",
           "mlora_plan_upload", "mlora_forward", "mlora_backward", "mlora_adamw_step", "mlora_profile_enable",
           "mlora_profile_read", "mlora_device_check", "mlora_status_string", "mlora_last_error",
           "mlora_version", "mlora_base_transpose", "mlora_forward_noalloc"]


class PlanOpts(ctypes.Structure):
    _fields_ = [("nano_rows", ctypes.c_int32), ("gemm_rows", ctypes.c_int32),
                ("n_streams", ctypes.c_int32), ("chunk_min", ctypes.c_int32),
                ("chunk_max", ctypes.c_int32), ("chunk_per_rank", ctypes.c_int32),
                ("w0_layout", ctypes.c_int32), ("w0_format", ctypes.c_int32),
                ("act_format", ctypes.c_int32), ("wg_overlap", ctypes.c_int32),
                ("grad_accumulate", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("n", ctypes.c_int64), ("d_in", ctypes.c_int64),
                ("d_out", ctypes.c_int64), ("dtype", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("z_elems", ctypes.c_int64), ("z_bytes", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("table_bytes", ctypes.c_int64),
                ("rpad_total", ctypes.c_int64), ("partial_rows", ctypes.c_int64),
                ("n_nano", ctypes.c_int64), ("n_chunks", ctypes.c_int64),
                ("n_tiles", ctypes.c_int64), ("n_ext", ctypes.c_int64),
                ("n_opt_blocks", ctypes.c_int64), ("n_proj", ctypes.c_int64),
                ("act_offset", ctypes.c_int64), ("dz_offset", ctypes.c_int64),
                ("wg_side", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class AdamwHparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float), ("step", ctypes.c_int32),
                ("max_grad_norm", ctypes.c_float)]


class MloraError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmlora.so (built in-tree).  Raises if it has not been built:
    there is no fallback implementation."""
    global _lib
    if _lib is not None:
        return _lib
    try:  # bind to the HIP runtime torch ships, so streams and memory are shared
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with "
                          "`python -m adapter_lora_segments_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.mlora_plan.argtypes = [i32, ctypes.POINTER(i64), ctypes.POINTER(i32), i64, i64, i32,
                             ctypes.POINTER(PlanOpts), ctypes.POINTER(vp)]
    L.mlora_plan.restype = i32
    L.mlora_plan_from_ids.argtypes = [i32, i64, ctypes.POINTER(i32), ctypes.POINTER(i32), i64, i64, i32,
                                      ctypes.POINTER(PlanOpts), ctypes.POINTER(vp)]
    L.mlora_plan_from_ids.restype = i32
    L.mlora_plan_multi.argtypes = [i32, ctypes.POINTER(i64), i32, ctypes.POINTER(i64), ctypes.POINTER(i32),
                                   i64, i32, ctypes.POINTER(PlanOpts), ctypes.POINTER(vp)]
    L.mlora_plan_multi.restype = i32
    L.mlora_plan_multi_from_ids.argtypes = [i32, i64, ctypes.POINTER(i32), i32, ctypes.POINTER(i64),
                                            ctypes.POINTER(i32), i64, i32, ctypes.POINTER(PlanOpts),
                                            ctypes.POINTER(vp)]
    L.mlora_plan_multi_from_ids.restype = i32
    L.mlora_plan_destroy.argtypes = [vp]
    L.mlora_plan_destroy.restype = None
    L.mlora_base_transpose.restype = i32
    L.mlora_base_transpose.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int64, i32, vp]
    L.mlora_plan_get_info.argtypes = [vp, ctypes.POINTER(PlanInfo)]
    L.mlora_plan_get_info.restype = i32
    L.mlora_plan_export.argtypes = [vp, i32, vp, ctypes.POINTER(sz)]
    L.mlora_plan_export.restype = i32
    L.mlora_plan_upload.argtypes = [vp, vp, sz, vp]
    L.mlora_plan_upload.restype = i32
    L.mlora_forward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.mlora_forward.restype = i32
    L.mlora_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.mlora_forward_noalloc.restype = i32
    L.mlora_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.mlora_backward.restype = i32
    L.mlora_adamw_step.argtypes = [vp] + [vp] * 11 + [i32, vp, sz, vp]
    L.mlora_adamw_step.restype = i32
    L.mlora_profile_enable.argtypes = [vp, i32]
    L.mlora_profile_enable.restype = i32
    L.mlora_profile_read.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    L.mlora_profile_read.restype = i32
    L.mlora_device_check.argtypes = []
    L.mlora_device_check.restype = i32
    L.mlora_status_string.argtypes = [i32]
    L.mlora_status_string.restype = ctypes.c_char_p
    L.mlora_last_error.argtypes = []
    L.mlora_last_error.restype = ctypes.c_char_p
    L.mlora_version.argtypes = []
    L.mlora_version.restype = ctypes.c_char_p
    _lib = L
    return L


def check(status: int) -> None:
    if status != MLORA_OK:
        raise MloraError(status, lib().mlora_last_error().decode())
