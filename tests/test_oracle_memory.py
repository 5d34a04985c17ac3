"""Pins of the oracle's KV memory operations (decode-loop page, "Decode
loop: batching, KV cache, memory management", section "KV cache details";
engine page, Step 10, tokens of several sequences):

* the page's defrag figure, cell for cell (tests/golden/defrag_figure.txt);
* sequence-set bookkeeping of seq_cp / seq_keep / seq_rm on shared cells;
* invariances of the whole model: a prefix shared by two sequences, a
  prefix copied with seq_cp (one stream or between streams), a cache
  compacted by defrag and a cache after seq_keep give the same logits as
  separate single-sequence contexts decoding the same token lists (up to
  float64 rounding: only the order of the cells in the attention sums
  differs).
"""
import os

import numpy as np
import pytest

from oracle import Batch, OracleContext, OracleModel
from oracle.planner import KVMemory
from workloads import MODELS, gen_tensor, tensor_specs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "defrag_figure.txt")


def read_figure():
    part, out = None, {"before": [], "after": []}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line in out:
            part = line
            continue
        out[part].append([int(v) for v in line.split()])
    return out


def test_defrag_matches_the_page_figure():
    fig = read_figure()
    m = KVMemory(1, 7, unified=True, n_seq_max=2)
    for c, s, p in fig["before"]:
        if s >= 0:
            m.occupy(0, c, p, s)
    src = m.defrag()
    for c, s, p in fig["after"]:
        assert m.pos[0, c] == p
        assert m.has[0, c].tolist() == [s == 0, s == 1]
    assert src[0].tolist() == [0, 1, 4, 3, 6]
    assert (m.seq_pos_max(0), m.seq_pos_max(1), m.n_kv(0)) == (2, 1, 5)


def test_seq_cp_keep_rm_on_one_stream():
    m = KVMemory(1, 8, unified=True, n_seq_max=3)
    for c in range(4):
        m.occupy(0, c, c, 0)
    assert m.seq_cp(0, 1, 1, 3)                 # positions 1 and 2
    assert m.has[0, :4, 1].tolist() == [False, True, True, False]
    assert (m.seq_pos_min(1), m.seq_pos_max(1)) == (1, 2)
    assert m.seq_cp(0, 2, -1, -1)
    m.seq_rm(0, -1, -1)                        # cells stay while 1 or 2 hold them
    assert m.pos[0, :4].tolist() == [0, 1, 2, 3]
    assert m.seq_keep(1)
    assert m.pos[0, :4].tolist() == [-1, 1, 2, -1]
    assert m.has[0, 1].tolist() == [False, True, False]
    assert not m.seq_cp(0, 3, -1, -1) and not m.seq_keep(3)


def test_seq_cp_between_streams_copies_the_whole_stream():
    m = KVMemory(2, 8, unified=False)
    m.occupy(0, [2, 5], [0, 1], 0)
    m.occupy(1, [0], [7], 1)
    assert not m.seq_cp(0, 1, 0, -1)           # only the full range
    assert m.seq_cp(0, 1, -1, -1)
    assert m.pos[1].tolist() == m.pos[0].tolist()
    assert m.has[1, [2, 5], 1].all() and m.has[1, :, 1].sum() == 2 and not m.has[1, :, 0].any()
    assert (m.seq_pos_min(1), m.seq_pos_max(1)) == (0, 1)


@pytest.fixture(scope="module")
def tiny():
    shape = MODELS["tiny-f32"]
    tens = {s.name: gen_tensor(shape, s) for s in tensor_specs(shape)}
    return OracleModel(shape, tens, dtype=np.float64)


def solo(model, tokens):
    """Logits of the last token of a single-sequence context."""
    ctx = OracleContext(model, n_ctx=256, n_batch=256, n_ubatch=256, n_seq_max=1, type_k="f32", type_v="f32")
    assert ctx.decode(Batch(list(tokens))) == 0
    return ctx.logits_ith(-1)


def close(a, b):
    return np.abs(a - b).max() <= 1e-10 * np.abs(b).max()


P, A, B = [11, 22, 33, 44, 55], [66, 77], [88, 99, 111]


def ctx_of(model, n_seq, unified):
    return OracleContext(model, n_ctx=256, n_batch=256, n_ubatch=4, n_seq_max=n_seq, type_k="f32",
                         type_v="f32", kv_unified=unified)


def test_shared_prefix_equals_separate_sequences(tiny):
    ctx = ctx_of(tiny, 2, True)
    assert ctx.decode(Batch(P, seq_id=[[0, 1]] * len(P), logits=[0] * len(P))) == 0
    assert ctx.decode(Batch(A + B, seq_id=[0] * 2 + [1] * 3, logits=[0, 1, 0, 0, 1])) == 0
    assert close(ctx.logits_ith(1), solo(tiny, P + A))
    assert close(ctx.logits_ith(4), solo(tiny, P + B))


def test_shared_token_attends_to_its_first_sequence(tiny):
    ctx = ctx_of(tiny, 2, True)
    assert ctx.decode(Batch([A[0], B[0]], seq_id=[0, 1], logits=[0, 0])) == 0
    assert ctx.decode(Batch([P[0]], seq_id=[[0, 1]], pos=[2], logits=[1])) == -1
    assert ctx.decode(Batch([P[0]], seq_id=[[0, 1]], logits=[1])) == 0
    assert close(ctx.logits_ith(0), solo(tiny, [A[0], P[0]]))
    ctx2 = ctx_of(tiny, 2, True)
    assert ctx2.decode(Batch([A[0], B[0]], seq_id=[0, 1], logits=[0, 0])) == 0
    assert ctx2.decode(Batch([P[0]], seq_id=[[1, 0]], logits=[1])) == 0
    assert close(ctx2.logits_ith(0), solo(tiny, [B[0], P[0]]))


@pytest.mark.parametrize("unified", [True, False])
def test_seq_cp_then_continue(tiny, unified):
    ctx = ctx_of(tiny, 2, unified)
    assert ctx.decode(Batch(P, seq_id=[0] * len(P))) == 0
    assert not ctx.seq_cp(0, 1, 2, -1) if not unified else True
    assert ctx.seq_cp(0, 1, -1, -1)
    assert ctx.decode(Batch(B, seq_id=[1] * 3)) == 0
    assert close(ctx.logits_ith(-1), solo(tiny, P + B))
    assert ctx.decode(Batch(A, seq_id=[0] * 2)) == 0
    assert close(ctx.logits_ith(-1), solo(tiny, P + A))


def test_defrag_and_keep_leave_the_logits_alone(tiny):
    ctx = ctx_of(tiny, 3, True)
    toks = P + A + B
    seq = [0, 1, 2, 0, 1, 2, 0, 1, 2, 0]
    assert ctx.decode(Batch(toks, seq_id=seq, logits=[0] * len(toks))) == 0
    ctx.seq_rm(1, -1, -1)
    ctx.seq_rm(2, 1, -1)
    moved = ctx.defrag()
    assert moved > 0
    assert ctx.mem.n_kv(0) == 4 + 1
    t0 = [toks[i] for i in range(len(toks)) if seq[i] == 0]
    assert ctx.decode(Batch([5], seq_id=[0])) == 0
    assert close(ctx.logits_ith(-1), solo(tiny, t0 + [5]))
    assert ctx.seq_keep(2)
    assert ctx.seq_pos_max(0) == -1 and ctx.seq_pos_max(2) == 0
    assert ctx.decode(Batch([6], seq_id=[2])) == 0
    assert close(ctx.logits_ith(-1), solo(tiny, [toks[2], 6]))
