"""Chained greedy generation (ubd_greedy_chain) through the C ABI on the
tiny f32 model: the picks equal the oracle's free-running greedy ids and
the step-by-step decode + greedy path's, with the same KV cells and the
same last logits; a chain longer than one block of picks; a chain that
runs out of KV cells part-way; an invalid first token."""
import numpy as np
import pytest

from oracle import OracleModel, OracleContext, Batch
from workloads import WORKLOADS, gen_tensor, tensor_specs, prompt_tokens

pytestmark = pytest.mark.gpu
BLOCK = 256         # UBD_GREEDY_CHAIN_BLOCK


@pytest.fixture(scope="module")
def tiny():
    import torch
    from llama_decode_ubatch_amd import Model
    assert torch.cuda.is_available()
    shape = WORKLOADS[1].model
    tens = {s.name: gen_tensor(shape, s) for s in tensor_specs(shape)}
    model = Model(shape, tens, device=0)
    om = OracleModel(shape, tens, dtype=np.float64)
    return shape, model, om


def prefilled(model, prompt, **kw):
    from llama_decode_ubatch_amd import Context
    ctx = Context(model, **kw)
    assert ctx.decode(prompt) == 0
    return ctx


def step_by_step(ctx, first, n):
    tok, ids = first, []
    for _ in range(n):
        assert ctx.decode([tok]) == 0
        tok = ctx.greedy(-1)
        ids.append(tok)
    return ids


@pytest.mark.parametrize("kv", ["f32", "f16"])
def test_chain_equals_oracle_and_step_by_step(tiny, kv):
    shape, model, om = tiny
    kw = dict(n_ctx=512, n_batch=512, n_ubatch=512, n_seq_max=1, type_k=kv, type_v=kv)
    prompt = prompt_tokens(WORKLOADS[1], 0)
    n = 24
    print(f"chain of {n} steps, {kv} KV", flush=True)
    a, b = prefilled(model, prompt, **kw), prefilled(model, prompt, **kw)
    ref = OracleContext(om, **kw)
    assert ref.decode(Batch(prompt)) == 0
    first = a.greedy(-1)
    assert first == b.greedy(-1) == ref.greedy(-1)

    ids = a.greedy_chain(first, n)
    steps = step_by_step(b, first, n)
    tok, oracle_ids = first, []
    for _ in range(n):
        assert ref.decode(Batch([tok])) == 0
        tok = ref.greedy(-1)
        oracle_ids.append(tok)

    assert ids.tolist() == steps
    assert ids.tolist() == oracle_ids
    assert a.seq_pos_max(0) == b.seq_pos_max(0) == prompt.size + n - 1
    assert np.array_equal(a.kv_cells(1), b.kv_cells(1))
    # the same kernels on the same inputs: the last step's logits are identical
    assert np.array_equal(a.logits_ith(-1), b.logits_ith(-1))
    # the context decodes on normally after a chain
    assert a.decode([int(ids[-1])]) == 0 and b.decode([int(ids[-1])]) == 0
    assert a.greedy(-1) == b.greedy(-1)


def test_chain_longer_than_one_block(tiny):
    shape, model, om = tiny
    kw = dict(n_ctx=512, n_batch=512, n_ubatch=512, n_seq_max=1, type_k="f16", type_v="f16")
    prompt = prompt_tokens(WORKLOADS[1], 1)
    n = BLOCK + 44
    print(f"chain of {n} steps", flush=True)
    a, b = prefilled(model, prompt, **kw), prefilled(model, prompt, **kw)
    first = a.greedy(-1)
    assert first == b.greedy(-1)
    ids = a.greedy_chain(first, n)
    assert ids.size == n
    assert ids.tolist() == step_by_step(b, first, n)


def test_chain_stops_when_the_cache_is_full(tiny):
    from llama_decode_ubatch_amd import last_error
    shape, model, om = tiny
    kw = dict(n_ctx=64, n_batch=64, n_ubatch=64, n_seq_max=1, type_k="f16", type_v="f16")
    prompt = prompt_tokens(WORKLOADS[1], 2)
    a, b = prefilled(model, prompt, **kw), prefilled(model, prompt, **kw)
    room = a.n_ctx - prompt.size
    print(f"n_ctx {a.n_ctx}: room for {room} steps", flush=True)
    assert 0 < room < BLOCK
    first = a.greedy(-1)
    ids = a.greedy_chain(first, room + 5)
    assert ids.size == room
    assert last_error()
    assert ids.tolist() == step_by_step(b, first, room)
    assert a.seq_pos_max(0) == prompt.size + room - 1


def test_chain_rejects_an_invalid_first_token(tiny):
    shape, model, om = tiny
    kw = dict(n_ctx=256, n_batch=256, n_ubatch=256, n_seq_max=1, type_k="f16", type_v="f16")
    a = prefilled(model, prompt_tokens(WORKLOADS[1], 3), **kw)
    with pytest.raises(RuntimeError):
        a.greedy_chain(shape.n_vocab, 4)
    assert a.greedy_chain(a.greedy(-1), 0).size == 0
