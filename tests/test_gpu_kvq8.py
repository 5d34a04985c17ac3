"""q8_0 KV cache: quantisation at append / fill and attention over codes.

* The quantiser is bit-exact: rows written through ubd_kv_fill (f32 and f16
  sources) and read back equal the oracle's q8_0 round trip of the same
  rows, value for value.
* The tiny model with a q8_0 cache, teacher-forced on the oracle's tokens:
  logits within 2e-3 of the max-norm.  The oracle quantises K / V computed
  in float64, the GPU the same rows computed in float32, so a code can land
  one step apart where a value sits on a rounding boundary; the bound
  covers that.
* The 8B shape with a q8_0 cache: sampled layers against the oracle's layer
  run from the GPU's own input and (decode) the GPU's dequantised KV prefix.
"""
import dataclasses

import numpy as np
import pytest

from oracle import Batch
from oracle import numerics as nm
from workloads import WORKLOADS, MODELS, gen_tensor, tensor_specs, prompt_tokens
from tests.helpers import oracle_ctx, oracle_layer_check

pytestmark = pytest.mark.gpu


def rel(a, b):
    return float(np.abs(np.asarray(a, np.float64) - b).max() / np.abs(b).max())


@pytest.fixture(scope="module")
def tiny():
    import torch  # noqa: F401
    from llama_decode_ubatch_amd import Model
    shape = MODELS["tiny-f32"]
    tens = {s.name: gen_tensor(shape, s) for s in tensor_specs(shape)}
    return shape, tens, Model(shape, tens, device=0)


def test_kv_fill_quantises_like_the_oracle(tiny):
    from llama_decode_ubatch_amd import Context
    shape, _, model = tiny
    ctx = Context(model, n_ctx=512, n_batch=512, n_ubatch=512, n_seq_max=1, type_k="q8_0", type_v="q8_0")
    rng = np.random.default_rng(11)
    n, ne, L = 200, shape.n_embd_kv, shape.n_layer
    scale = rng.uniform(1e-3, 30.0, (n, 1)).astype(np.float32)
    K = [(rng.standard_normal((n, ne)) * scale).astype(np.float32) for _ in range(L)]
    V = [(rng.standard_normal((n, ne)) * scale).astype(np.float32) for _ in range(L)]
    K[0][5] = 0.0                       # an all-zero row: zero scale, zero codes
    assert ctx.kv_fill(0, n, K, V, "f32") == 0
    for il in (0, L - 1):
        np.testing.assert_array_equal(ctx.kv_read(il, 0, 0, 0, n), nm.round_to_kv_type(K[il], "q8_0"))
        np.testing.assert_array_equal(ctx.kv_read(il, 0, 1, 0, n), nm.round_to_kv_type(V[il], "q8_0"))
    # f16 sources are quantised from their exact f32 values
    ctx.seq_rm(0, -1, -1)
    K16 = [k.astype(np.float16) for k in K]
    V16 = [v.astype(np.float16) for v in V]
    assert ctx.kv_fill(0, n, [k.view(np.uint16) for k in K16], [v.view(np.uint16) for v in V16], "f16") == 0
    np.testing.assert_array_equal(ctx.kv_read(1, 0, 0, 0, n), nm.round_to_kv_type(K16[1].astype(np.float32), "q8_0"))
    np.testing.assert_array_equal(ctx.kv_read(2, 0, 1, 0, n), nm.round_to_kv_type(V16[2].astype(np.float32), "q8_0"))


@pytest.mark.parametrize("n_seqs", [1, 4])
def test_tiny_model_q8_cache_teacher_forced(tiny, n_seqs):
    from llama_decode_ubatch_amd import Context
    shape, tens, model = tiny
    ctx = Context(model, n_ctx=1024, n_batch=512, n_ubatch=64, n_seq_max=n_seqs, type_k="q8_0", type_v="q8_0")
    ref = oracle_ctx(shape, tens, np.float64, n_ctx=1024, n_batch=512, n_ubatch=64, n_seq_max=n_seqs,
                     type_k="q8_0", type_v="q8_0")
    rng = np.random.default_rng(100 + n_seqs)
    n_p = 40
    toks = rng.integers(0, shape.n_vocab, n_p * n_seqs).astype(np.int32)
    seqs = np.repeat(np.arange(n_seqs), n_p).astype(np.int32)
    flags = np.zeros(n_p * n_seqs, np.int8)
    flags[n_p - 1::n_p] = 1
    assert ctx.decode(toks, seq_id=seqs, logits=flags) == 0
    assert ref.decode(Batch(toks, seq_id=seqs, logits=flags)) == 0
    errs = []
    for step in range(4):
        z = ctx.logits()
        zr = np.stack([ref.logits_ith(i) for i in np.nonzero(flags)[0]])
        errs.append(rel(z, zr))
        nxt = np.argmax(zr, axis=1).astype(np.int32)
        flags = np.ones(n_seqs, np.int8)
        assert ctx.decode(nxt, seq_id=np.arange(n_seqs), logits=flags) == 0
        assert ref.decode(Batch(nxt, seq_id=np.arange(n_seqs), logits=flags)) == 0
    print(f"tiny q8_0 cache, {n_seqs} seqs: logits rel err per step {['%.1e' % e for e in errs]}", flush=True)
    assert max(errs) < 2e-3


def test_8b_q8_cache_sampled_layers():
    import torch
    from llama_decode_ubatch_amd import Model, Context
    from oracle import OracleModel
    from workloads import device as wdev, gen_tensor_rows
    w = dataclasses.replace(WORKLOADS[3], type_k="q8_0", type_v="q8_0")
    tens = wdev.model_tensors(torch, w.model, "cuda:0")
    torch.cuda.synchronize()
    model = Model(w.model, tens, device=0)
    del tens
    torch.cuda.empty_cache()
    om = OracleModel(w.model, lambda n: gen_tensor(w.model, n), dtype=np.float32, cache=True,
                     rows_fn=lambda n, r: gen_tensor_rows(w.model, n, r))
    ctx = Context(model, n_ctx=w.n_ctx, n_batch=w.n_batch, n_ubatch=w.n_ubatch, type_k="q8_0", type_v="q8_0")
    assert ctx.keep_residuals(True) == 0
    prompt = prompt_tokens(w, 0)[:300]
    T = prompt.size
    assert ctx.decode(prompt) == 0
    for il in (0, 31):
        y, _ = oracle_layer_check(om, w, il, ctx.residual(il, T), prompt, 0)
        err = rel(ctx.residual(il + 1, T), y)
        print(f"  q8_0 cache prefill layer {il}: rel err {err:.2e}", flush=True)
        assert err < 3e-2
    tok = ctx.greedy(-1)
    assert ctx.decode([tok]) == 0
    for il in (0, 17):
        K = ctx.kv_read(il, 0, 0, 0, T)
        V = ctx.kv_read(il, 0, 1, 0, T)
        y, _ = oracle_layer_check(om, w, il, ctx.residual(il, 1), [tok], T, (K, V))
        err = rel(ctx.residual(il + 1, 1), y)
        print(f"  q8_0 cache decode layer {il}: rel err {err:.2e}", flush=True)
        assert err < 3e-2
    om.drop_cache()
