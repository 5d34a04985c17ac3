"""Pins for oracle/planner.py: the pages' stated rules for batch autofill,
validation, ubatch splitting, slot preparation and rollback (CPU only)."""
import numpy as np
import pytest

from oracle.planner import (Batch, KVMemory, plan_batch, sanitize,
                            split_equal, split_simple, rollback_ubatch,
                            context_geometry, RC_OK, RC_NO_SLOT, RC_INVALID)


def mem1(n=16):
    return KVMemory(1, n, unified=False)


def test_autofill_defaults():
    # engine page, Step 10: no seq ids -> sequence 0; no positions ->
    # seq_pos_max(s)+1 onward; no output flags -> last token only
    m = mem1()
    rc, sb = sanitize(Batch([5, 6, 7]), 100, 1, 64, m)
    assert rc == RC_OK
    assert sb.seq.tolist() == [0, 0, 0]
    assert sb.pos.tolist() == [0, 1, 2]
    assert sb.output.tolist() == [False, False, True]
    p = plan_batch(Batch([5, 6, 7]), m, 100, 1, 64, 64)
    for ub, c in zip(p.ubatches, p.cells):
        m.apply(ub, c)
    rc, sb = sanitize(Batch([9, 9]), 100, 1, 64, m)
    assert sb.pos.tolist() == [3, 4]


def test_autofill_positions_per_sequence():
    m = KVMemory(1, 32, unified=True)
    m.occupy(0, [0, 1, 2], [0, 1, 2], 1)
    rc, sb = sanitize(Batch([1, 2, 3, 4, 5], seq_id=[0, 1, 0, 1, 1]), 10, 2, 64, m)
    assert sb.pos.tolist() == [0, 3, 1, 4, 5]


@pytest.mark.parametrize("batch", [
    Batch([]),                                     # n_tokens <= 0
    Batch([1] * 65),                               # > n_batch
    Batch([100]),                                  # token >= n_vocab
    Batch([-1]),                                   # token < 0
    Batch([1, 2], seq_id=[0, 4]),                  # seq id >= n_seq_max
    Batch([1, 2], seq_id=[0, -1]),
    Batch([1], seq_id=[[0, 0]], n_seq_id=[2]),     # a sequence twice
    Batch([1], seq_id=[[0, 1]], n_seq_id=[0]),     # no sequence
    Batch([1], seq_id=[[0, 1]], n_seq_id=[3]),     # fewer ids than n_seq_id
    Batch([1, 2], pos=[0, 2]),                     # non-consecutive
    Batch([1, 2], pos=[1, 0]),
    Batch([1], pos=[-3]),
    Batch([1], embd=np.zeros(4)),                  # embeddings input
])
def test_invalid_batches(batch):
    m = mem1()
    assert plan_batch(batch, m, 100, 4, 64, 16).rc == RC_INVALID


def test_positions_must_continue_sequence():
    m = mem1()
    m.occupy(0, [0, 1], [0, 1], 0)
    assert plan_batch(Batch([1], pos=[3]), m, 100, 1, 64, 16).rc == RC_INVALID
    assert plan_batch(Batch([1], pos=[2]), m, 100, 1, 64, 16).rc == RC_OK
    # an empty sequence may start anywhere
    assert plan_batch(Batch([1, 2], pos=[7, 8], seq_id=[1, 1]),
                      KVMemory(1, 16, True), 100, 2, 64, 16).rc == RC_OK


def test_split_simple_chunks():
    rc, sb = sanitize(Batch(list(range(10))), 100, 1, 64, mem1())
    ubs = split_simple(sb, 4)
    assert [u.idx.tolist() for u in ubs] == [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9]]


def test_split_equal_config2_shapes():
    # 8 sequences x 128 tokens, seq-major, n_ubatch 128 -> 8 ubatches of 8 x 16
    seq = np.repeat(np.arange(8), 128)
    m = KVMemory(8, 256, unified=False)
    logits = np.zeros(1024, np.int8); logits[127::128] = 1
    rc, sb = sanitize(Batch(np.ones(1024, int), seq_id=seq, logits=logits), 200, 8, 1024, m)
    ubs = split_equal(sb, 128)
    assert len(ubs) == 8
    for k, u in enumerate(ubs):
        assert (u.n_seqs, u.n_seq_tokens, u.n_tokens) == (8, 16, 128)
        assert u.seq.tolist() == list(np.repeat(np.arange(8), 16))
        assert u.pos.tolist() == list(np.tile(np.arange(16 * k, 16 * k + 16), 8))
    # all outputs fall in the last ubatch
    assert [int(u.output.sum()) for u in ubs] == [0] * 7 + [8]
    # one token per sequence (decode) -> a single ubatch
    rc, sb = sanitize(Batch(np.ones(8, int), seq_id=np.arange(8)), 200, 8, 1024, m)
    assert [u.n_tokens for u in split_equal(sb, 128)] == [8]


def test_split_equal_uneven_and_order():
    m = KVMemory(3, 64, unified=False)
    seq = [2, 0, 2, 2, 0, 1, 2]
    rc, sb = sanitize(Batch(list(range(7)), seq_id=seq), 100, 3, 64, m)
    ubs = split_equal(sb, 6)
    # first appearance order 2, 0, 1; min remaining 1 -> k = 1
    assert ubs[0].idx.tolist() == [0, 1, 5]
    assert ubs[1].idx.tolist() == [2, 4]        # seqs 2, 0 left: k = min(2, 1, 3) = 1
    assert ubs[2].idx.tolist() == [3, 6]        # only seq 2: k = min(2, 6)
    assert sum(u.n_tokens for u in ubs) == 7


def test_slots_lowest_free_and_prepare_all_or_nothing():
    m = mem1(8)
    m.occupy(0, [1, 4], [0, 1], 0)
    p = plan_batch(Batch([1, 2, 3]), m, 10, 1, 64, 2)
    assert [c.tolist() for c in p.cells] == [[0, 2], [3]]
    # 6 free cells; a 7-token batch needs 7 -> return 1 with the cells as
    # they were (compaction would keep 6 free cells, so no retry)
    pos0, has0 = m.pos.copy(), m.has.copy()
    p = plan_batch(Batch([1] * 7), m, 10, 1, 64, 2)
    assert p.rc == RC_NO_SLOT
    assert np.array_equal(m.pos, pos0) and np.array_equal(m.has, has0)
    assert m.pos[0].tolist() == [-1, 0, -1, -1, 1, -1, -1, -1]
    assert (m.seq_pos_min(0), m.seq_pos_max(0)) == (0, 1)


def test_shared_tokens_need_a_unified_cache():
    assert plan_batch(Batch([1], seq_id=[[0, 1]], n_seq_id=[2]), KVMemory(2, 16, False),
                      100, 2, 64, 16).rc == RC_INVALID
    m = KVMemory(1, 16, True, 4)
    p = plan_batch(Batch([1, 2, 3], seq_id=[[0, 1, 2], [0, 1, 2], [1]]), m, 100, 4, 64, 16)
    assert p.rc == RC_OK
    for ub, c in zip(p.ubatches, p.cells):
        m.apply(ub, c)
    # one cell per token; the shared ones hold all three sequences
    assert m.pos[0, :3].tolist() == [0, 1, 2]
    assert m.has[0, 0, :3].all() and m.has[0, 1, :3].all()
    assert m.has[0, 2].tolist() == [False, True, False, False]
    assert [m.seq_pos_max(s) for s in range(4)] == [1, 2, 1, -1]
    # positions continue each sequence of a shared token
    assert plan_batch(Batch([5], seq_id=[[0, 1]]), m, 100, 4, 64, 16).rc == RC_INVALID
    assert plan_batch(Batch([5], seq_id=[[0, 2]]), m, 100, 4, 64, 16).rc == RC_OK
    assert plan_batch(Batch([5], pos=[2], seq_id=[[0, 2]]), m, 100, 4, 64, 16).rc == RC_OK
    assert plan_batch(Batch([5], pos=[2], seq_id=[[0, 1]]), m, 100, 4, 64, 16).rc == RC_INVALID
    # a shared cell stays until its last sequence leaves it
    m.seq_rm(0, -1, -1)
    assert m.pos[0, :3].tolist() == [0, 1, 2] and not m.has[0, :, 0].any()
    m.seq_rm(1, -1, -1)
    m.seq_rm(2, 1, -1)
    assert m.pos[0, :3].tolist() == [0, -1, -1] and m.has[0, 0].tolist() == [False, False, True, False]


def test_seq_rm_and_reuse():
    m = mem1(8)
    p = plan_batch(Batch([1] * 6), m, 10, 1, 64, 8)
    m.apply(p.ubatches[0], p.cells[0])
    assert (m.seq_pos_min(0), m.seq_pos_max(0)) == (0, 5)
    m.seq_rm(0, 2, 4)
    assert m.pos[0].tolist() == [0, 1, -1, -1, 4, 5, -1, -1]
    m.seq_rm(0, 5, -1)
    assert m.seq_pos_max(0) == 4
    m.seq_rm(-1, -1, -1)
    assert m.seq_pos_max(0) == -1 and m.n_kv(0) == 0


def test_rollback_removes_from_pos_min():
    m = KVMemory(1, 32, unified=True)
    p = plan_batch(Batch([1] * 6, seq_id=[0, 1, 0, 1, 0, 1]), m, 10, 2, 64, 2)
    for ub, c in zip(p.ubatches[:2], p.cells[:2]):
        m.apply(ub, c)
    m.apply(p.ubatches[2], p.cells[2])
    rollback_ubatch(m, p.ubatches[2])
    assert (m.seq_pos_max(0), m.seq_pos_max(1)) == (1, 1)


def test_output_rows_in_batch_order():
    m = KVMemory(2, 16, unified=False)
    p = plan_batch(Batch([1, 2, 3, 4], seq_id=[1, 0, 1, 0], logits=[1, 0, 1, 1]),
                   m, 10, 2, 64, 16)
    assert p.out_row.tolist() == [0, -1, 1, 2] and p.n_outputs == 3


def test_context_geometry_padding():
    # n_ctx is padded to a multiple of 256 and split across streams
    assert context_geometry(4096, 1, False) == (4096, 1, 4096)
    assert context_geometry(1000, 1, False) == (1024, 1, 1024)
    assert context_geometry(2048, 8, False) == (2048, 8, 256)
    assert context_geometry(2048, 8, True) == (2048, 1, 2048)
    assert context_geometry(16 * 32768, 16, False)[2] == 32768
