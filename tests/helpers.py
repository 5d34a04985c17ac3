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


def oracle_layer_check(om, w, il, x_in, tokens, pos0=0, kv_prefix=None):
    """The oracle's layer `il` for one sequence's tokens at positions
    pos0.. given the residual entering the layer (x_in, from the GPU) and,
    for pos0 > 0, the f16 K/V rows of positions < pos0 (from the GPU cache).
    Only layer il's KV storage is allocated.  Returns (x_out, context)."""
    from oracle import OracleContext, Batch
    from oracle.planner import plan_batch
    n_ctx = pos0 + max(256, len(tokens))
    ref = OracleContext(om, n_ctx=n_ctx, n_batch=n_ctx, n_ubatch=n_ctx, n_seq_max=1,
                        type_k=w.type_k, type_v=w.type_v)
    if pos0:
        cells = ref.mem.fill_sequence(0, pos0)
        K, V = ref.kv(il, 0)
        K[cells] = kv_prefix[0]
        V[cells] = kv_prefix[1]
    plan = plan_batch(Batch(np.asarray(tokens)), ref.mem, w.model.n_vocab, 1, ref.n_batch, len(tokens))
    ub, cells = plan.ubatches[0], plan.cells[0]
    ref.mem.apply(ub, cells)
    y = ref.layer_forward(il, np.asarray(x_in, np.float32), ub, cells)
    for k in [k for k in om._cache if k.startswith(f"blk.{il}.")]:
        del om._cache[k]
    return y, ref
