"""Packed multi-LoRA linear layer (forward and backward) for AMD MI355X.

The compute lives in ``libmlora.so`` (HIP, gfx950, built in-tree by
``adapter_lora_segments_amd.build``); this package only marshals arguments.
Importing the binding does not load the library; the first call does, and
fails loudly if it has not been built.
"""
from .binding import (Plan, PackedLoRALinear, AdamW, mlora_plan, mlora_forward,  # noqa: F401
                      mlora_backward, mlora_adamw_step, adamw_hparams, pointer_table, device_check,
                      base_both, mlora_base_transpose, mlora_forward_noalloc)
from ._lib import MloraError, lib  # noqa: F401
