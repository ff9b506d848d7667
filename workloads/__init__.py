"""Seeded synthetic inputs for the multi-LoRA linear layer.

This package is the one piece shared by the oracle side (tests, oracle timing)
and the device side (tests, bench).  It draws integers (token counts, ranks)
and tensor values and nothing else: it holds none of the layer's arithmetic.

- ``configs``  the five workloads (shapes, adapter counts, rank sets, token
               count distributions) and their frozen integer structure;
- ``tensors``  seeded tensor values, rounded to bf16 (round-to-nearest-even)
               on the host so both sides see identical bits.
"""
from .configs import Workload, Projection, load_workload, WORKLOAD_NAMES  # noqa: F401
