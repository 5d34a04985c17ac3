"""Seeded synthetic inputs shared by the oracle and the GPU path.

This package holds only input *generation*: model shapes, the five workloads,
and a counter-based generator that fills any slice of any weight tensor,
prompt or KV pre-fill block identically on the host (NumPy, here) and on the
device (``workloads/synth.hip``).  It contains none of the transformer's
arithmetic; both the oracle and the HIP path import it, and it imports
neither of them.
"""
from .configs import (MODELS, WORKLOADS, ModelShape, Workload, tensor_specs,
                      TensorSpec)
from .gen import (SEED, mix64, tensor_key, prompt_key, kv_key, hashes,
                  normal_table_f32, normal_table_bf16, gain_table_f32,
                  kv_table_f16, gen_tensor, gen_tensor_rows, prompt_tokens,
                  kv_prefill_block, q8_codes_from_hash, q8_scale_bits_from_hash)

__all__ = [
    "MODELS", "WORKLOADS", "ModelShape", "Workload", "tensor_specs",
    "TensorSpec", "SEED", "mix64", "tensor_key", "prompt_key", "kv_key",
    "hashes", "normal_table_f32", "normal_table_bf16", "gain_table_f32",
    "kv_table_f16", "gen_tensor", "gen_tensor_rows", "prompt_tokens",
    "kv_prefill_block", "q8_codes_from_hash", "q8_scale_bits_from_hash",
]
