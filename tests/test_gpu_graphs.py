"""Decode-step graphs (graph_reuse): the first ubatch of a shape is captured
as a HIP graph and later ubatches of that shape replay it.  Every replay is
compared bit for bit with a context that launches kernel by kernel
(graph_reuse = False) on the same inputs, with host reads of the logits and
greedy picks (synchronising the stream) between replays, and the capture and
reuse counters of ubd_perf are checked.  The engine page's Step 13a
describes the reuse; the architecture page's Example 15 prints its counter
for a 4-token prompt and 8 new tokens (one prompt decode and 7 one-token
decodes): 6 graphs reused.
"""
import numpy as np
import pytest

from workloads import WORKLOADS, ModelShape, gen_tensor, tensor_specs
from tests.helpers import rand_tokens

pytestmark = pytest.mark.gpu

# head size 32, f16 KV: the MFMA attention, split over cells for <= 16 tokens
SMALL = ModelShape("small-bf16-a", 10, n_layer=2, n_embd=256, n_head=8, n_head_kv=2, n_ff=1408,
                   n_vocab=1024, n_ctx_train=2048, rope_base=10000.0, wtype="bf16")


@pytest.fixture(scope="module")
def small():
    import torch  # noqa: F401
    from llama_decode_ubatch_amd import Model
    tens = {s.name: gen_tensor(SMALL, s) for s in tensor_specs(SMALL)}
    return Model(SMALL, tens, device=0)


def pair(model, **kw):
    from llama_decode_ubatch_amd import Context
    return (Context(model, graph_reuse=True, **kw), Context(model, graph_reuse=False, **kw))


def step_both(cg, ce, tokens, **kw):
    assert cg.decode(tokens, **kw) == 0 and ce.decode(tokens, **kw) == 0
    zg, ze = cg.logits(), ce.logits()
    assert np.array_equal(zg, ze)
    return zg


def test_prefill_and_decode_replays_equal_eager(small):
    """250-token prefill, then 12 one-token steps whose scans (251..262
    cells) fall in two 256-cell buckets: three shapes captured, the other
    10 steps replayed."""
    cg, ce = pair(small, n_ctx=1024, n_batch=512, n_ubatch=512)
    prompt = rand_tokens(250, SMALL.n_vocab, seed=71)
    step_both(cg, ce, prompt)
    for step in range(12):
        tok = ce.greedy(-1)
        assert cg.greedy(-1) == tok
        step_both(cg, ce, [tok])
    pg, pe = cg.perf(), ce.perf()
    print(f"graphs captured {pg['n_graphs']}, reused {pg['n_reused']}", flush=True)
    assert (pg["n_graphs"], pg["n_reused"], pg["n_ubatch"]) == (3, 10, 13)
    assert (pe["n_graphs"], pe["n_reused"], pe["n_ubatch"]) == (0, 0, 13)
    cg.free()
    ce.free()


def test_four_sequences_replays_equal_eager(small):
    """Four sequences prefilled in one batch, then one token per sequence per
    step (4-token ubatches, all rows flagged) for 6 steps."""
    cg, ce = pair(small, n_ctx=2048, n_batch=512, n_ubatch=512, n_seq_max=4)
    n = 40
    toks = np.concatenate([rand_tokens(n, SMALL.n_vocab, seed=80 + s) for s in range(4)])
    seq = np.repeat(np.arange(4), n)
    pos = np.tile(np.arange(n), 4)
    logits = np.zeros(4 * n, np.int8)
    logits[n - 1::n] = 1
    step_both(cg, ce, toks, pos=pos, seq_id=seq, logits=logits)
    for step in range(6):
        nxt = np.array([int(np.argmax(ce.logits_ith(i))) for i in range(4)], np.int32)
        step_both(cg, ce, nxt, pos=np.full(4, n + step), seq_id=np.arange(4), logits=np.ones(4, np.int8))
    pg = cg.perf()
    assert (pg["n_graphs"], pg["n_reused"]) == (2, 5)
    cg.free()
    ce.free()


def test_tuning_change_recaptures(small):
    """A kernel-choice change drops the captured graphs: the next step is
    captured again with the new choice, and still equals the eager
    context."""
    from llama_decode_ubatch_amd.binding import set_tuning
    cg, ce = pair(small, n_ctx=512, n_batch=512, n_ubatch=512)
    step_both(cg, ce, rand_tokens(20, SMALL.n_vocab, seed=90))
    tok = ce.greedy(-1)
    for _ in range(3):
        step_both(cg, ce, [tok])
    assert (cg.perf()["n_graphs"], cg.perf()["n_reused"]) == (2, 2)
    try:
        set_tuning("ldsx_early", 0)
        for _ in range(3):
            step_both(cg, ce, [tok])
        assert (cg.perf()["n_graphs"], cg.perf()["n_reused"]) == (3, 4)
    finally:
        set_tuning("ldsx_early", 1)
    step_both(cg, ce, [tok])
    assert cg.perf()["n_graphs"] == 4
    cg.free()
    ce.free()


def test_example_counter_six_reused_for_seven_decodes():
    """Architecture page, Example 15: the tiny model with a 4-token prompt and
    8 new tokens runs one prompt decode and 7 one-token decodes of one
    shape, 6 of which reuse the graph.  The greedy tokens also follow the
    oracle's."""
    import torch  # noqa: F401
    from llama_decode_ubatch_amd import Model, Context
    from oracle import OracleModel, OracleContext, Batch
    shape = WORKLOADS[1].model
    tens = {s.name: gen_tensor(shape, s) for s in tensor_specs(shape)}
    model = Model(shape, tens, device=0)
    kw = dict(n_ctx=256, n_batch=256, n_ubatch=256, type_k="f32", type_v="f32")
    cg, ce = Context(model, **kw), Context(model, graph_reuse=False, **kw)
    ref = OracleContext(OracleModel(shape, tens, dtype=np.float64), **kw)
    prompt = rand_tokens(4, shape.n_vocab, seed=95)
    step_both(cg, ce, prompt)
    assert ref.decode(Batch(prompt)) == 0
    new = []
    for i in range(8):
        tok = cg.greedy(-1)
        assert tok == ref.greedy(-1)
        new.append(tok)
        if i == 7:
            break
        step_both(cg, ce, [tok])
        assert ref.decode(Batch([tok])) == 0
    p = cg.perf()
    print(f"{len(new)} new tokens, {p['n_decode']} decode runs, graphs reused = {p['n_reused']}", flush=True)
    assert (p["n_decode"], p["n_reused"]) == (8, 6)
    cg.free()
    ce.free()
    model.free()
