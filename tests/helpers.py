"""Shared test helpers: small model shapes and oracle construction."""
import numpy as np

from workloads import ModelShape, gen_tensor, tensor_specs

# A small Llama-architecture shape for fast invariant tests (same structure as
# the tiny model: GQA with 2 KV heads, SwiGLU, untied output).
MICRO = ModelShape("micro", 9, n_layer=2, n_embd=64, n_head=4, n_head_kv=2,
                   n_ff=96, n_vocab=300, n_ctx_train=512, rope_base=10000.0,
                   wtype="f32")


def micro_tensors(shape=MICRO):
    return {s.name: gen_tensor(shape, s) for s in tensor_specs(shape)}


def oracle_ctx(shape=MICRO, tensors=None, dtype=np.float64, **kw):
    from oracle import OracleModel, OracleContext
    tensors = tensors if tensors is not None else micro_tensors(shape)
    m = OracleModel(shape, tensors, dtype=dtype)
    kw.setdefault("n_ctx", 256)
    kw.setdefault("type_k", "f32")
    kw.setdefault("type_v", "f32")
    return OracleContext(m, **kw)


def rand_tokens(n, vocab, seed):
    return np.random.default_rng(seed).integers(0, vocab, n).astype(np.int32)
