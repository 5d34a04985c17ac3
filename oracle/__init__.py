"""Parity oracle: a plain, slow, CPU forward of one ``llama_decode`` step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP path (``llama_decode_ubatch_amd``); the only common dependency is the
seeded input generator in ``workloads/``.

What it computes, and where the pages define it:
  * ``numerics``  RMSNorm, RoPE (normal pairing), SwiGLU, softmax attention,
                  32-element int8 block dequantisation, KV storage rounding.
  * ``planner``   batch validation and autofill, ubatch splitting, KV-cell
                  slot search / apply / removal, decode return codes.
  * ``model``     the per-ubatch Llama forward and the logits/greedy readout.

Parity status of each function is stated in its docstring; functions whose
values the pages do not print are pinned by closed forms, invariants and
brute force in ``tests/test_oracle_*.py``.
"""
from . import numerics, planner, model  # noqa: F401
from .planner import Batch, KVMemory, plan_batch  # noqa: F401
from .model import OracleModel, OracleContext  # noqa: F401
