"""Oracle for the packed multi-LoRA linear layer -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct CPU implementation in float64 (numpy), used
only by ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py``.  The product path (the HIP library and its Python binding) never
imports, calls or links anything here, and nothing here imports the product.

- ``lora``        per-adapter LoRA forward and backward (the plain definition);
- ``plan_mirror`` an independent re-implementation of the plan rule the
                  library's host plan builder follows, for bit-exact checks.

Sources: PLoRA: Efficient Concurrent LoRA Training for Large Language Models
(academ.us full text) §2.1 (LoRA shapes and scaled update), §2.4 (each packed
adapter computes exactly standard LoRA), §9.2 (concatenated adapters, token
axis = sequence x batch, the four backward cases).
"""
