"""KV memory operations on the GPU against the oracle (decode-loop page,
"Decode loop: batching, KV cache, memory management", section "KV cache
details"; engine page, Step 10, tokens of several sequences): the same
operations on both sides, then

* cell tables (position and sequence set of every cell) equal exactly;
* logits within 1e-4 of the max-norm (tiny f32 model; f16 caches are
  rounded the same way by the oracle), 2e-3 with q8_0 caches (a code can
  land one step apart where the float32 and float64 K / V rows straddle a
  rounding boundary);
* K/V rows moved by defrag or copied between streams are bit-exact copies
  of the rows read before.
"""
import numpy as np
import pytest

from oracle import OracleModel, OracleContext, Batch
from workloads import WORKLOADS, gen_tensor, tensor_specs

pytestmark = pytest.mark.gpu
TOL = 1e-4


def rel_err(z, zr):
    return float(np.abs(np.asarray(z, np.float64) - zr).max() / np.abs(zr).max())


@pytest.fixture(scope="module")
def tiny():
    import torch
    from llama_decode_ubatch_amd import Model
    assert torch.cuda.is_available()
    shape = WORKLOADS[1].model
    tens = {s.name: gen_tensor(shape, s) for s in tensor_specs(shape)}
    return shape, Model(shape, tens, device=0), OracleModel(shape, tens, dtype=np.float64)


def make(tiny, **kw):
    from llama_decode_ubatch_amd import Context
    _, model, om = tiny
    return Context(model, **kw), OracleContext(om, **kw)


def same_tables(ctx, ref):
    for st in range(ref.n_stream):
        pos, has = ctx.cells(st)
        assert pos.tolist() == ref.mem.pos[st].tolist(), st
        assert np.array_equal(has, ref.mem.has[st]), st


def decode_both(ctx, ref, toks, seq_id=None, logits=None, pos=None, tol=TOL):
    rc = ctx.decode(toks, seq_id=seq_id, logits=logits, pos=pos)
    assert rc == ref.decode(Batch(list(toks), seq_id=seq_id, logits=logits, pos=pos))
    same_tables(ctx, ref)
    if rc == 0:
        z = ctx.logits()
        zr = np.stack([ref.logits_ith(i) for i in range(len(toks)) if ref.out_row[i] >= 0])
        err = rel_err(z, zr)
        assert err < tol, err
    return rc


def read_kv(ctx, il, st, n):
    return ctx.kv_read(il, st, 0, 0, n), ctx.kv_read(il, st, 1, 0, n)


@pytest.mark.parametrize("kv", ["f32", "f16"])
def test_shared_prefix_tokens(tiny, kv):
    """A 40-token prefix shared by four sequences (one cell per token),
    then each sequence continues on its own."""
    shape = tiny[0]
    ctx, ref = make(tiny, n_ctx=1024, n_batch=256, n_ubatch=32, n_seq_max=4, kv_unified=True,
                    type_k=kv, type_v=kv)
    rng = np.random.default_rng(7)
    pre = rng.integers(0, shape.n_vocab, 40).tolist()
    print(f"shared prefix, {kv} cache", flush=True)
    flags = [0] * 39 + [1]
    assert decode_both(ctx, ref, pre, seq_id=[[0, 1, 2, 3]] * 40, logits=flags) == 0
    toks = rng.integers(0, shape.n_vocab, 4 * 6).tolist()
    seq = np.repeat(np.arange(4), 6).tolist()
    assert decode_both(ctx, ref, toks, seq_id=seq, logits=[1] * 24) == 0
    for step in range(3):
        nxt = [int(np.argmax(ref.logits_ith(i))) for i in range(4)] if step else \
            [int(np.argmax(ref.logits_ith(6 * i + 5))) for i in range(4)]
        assert decode_both(ctx, ref, nxt, seq_id=[0, 1, 2, 3], logits=[1] * 4) == 0
    # a token of several sequences needs a unified cache
    ctx2, ref2 = make(tiny, n_ctx=512, n_batch=64, n_ubatch=32, n_seq_max=2)
    assert ctx2.decode([1], seq_id=[[0, 1]]) == ref2.decode(Batch([1], seq_id=[[0, 1]])) == -1


@pytest.mark.parametrize("kv", ["f16", "q8_0"])
def test_seq_cp_between_streams_copies_rows(tiny, kv):
    shape = tiny[0]
    ctx, ref = make(tiny, n_ctx=3 * 256, n_batch=256, n_ubatch=64, n_seq_max=3, type_k=kv, type_v=kv)
    rng = np.random.default_rng(8)
    pre = rng.integers(0, shape.n_vocab, 70).tolist()
    print(f"seq_cp across streams, {kv} cache", flush=True)
    tol = 2e-3 if kv == "q8_0" else TOL
    assert decode_both(ctx, ref, pre, seq_id=[0] * 70, tol=tol) == 0
    assert not ctx.seq_cp(0, 1, 5, -1) and not ref.seq_cp(0, 1, 5, -1)
    for dst in (1, 2):
        assert ctx.seq_cp(0, dst, -1, -1) and ref.seq_cp(0, dst, -1, -1)
    same_tables(ctx, ref)
    for il in (0, shape.n_layer - 1):
        k0, v0 = read_kv(ctx, il, 0, 70)
        for st in (1, 2):
            k, v = read_kv(ctx, il, st, 70)
            assert np.array_equal(k, k0) and np.array_equal(v, v0)
    toks = rng.integers(0, shape.n_vocab, 3 * 4).tolist()
    assert decode_both(ctx, ref, toks, seq_id=np.repeat(np.arange(3), 4).tolist(), logits=[1] * 12, tol=tol) == 0


@pytest.mark.parametrize("kv,unified", [("f16", True), ("f32", False), ("q8_0", True)])
def test_defrag_moves_rows_and_keeps_logits(tiny, kv, unified):
    shape = tiny[0]
    n_seq = 3
    ctx, ref = make(tiny, n_ctx=n_seq * 256, n_batch=256, n_ubatch=48, n_seq_max=n_seq, kv_unified=unified,
                    type_k=kv, type_v=kv)
    rng = np.random.default_rng(9)
    print(f"defrag, {kv} cache, unified={unified}", flush=True)
    tol = 2e-3 if kv == "q8_0" else TOL
    toks = rng.integers(0, shape.n_vocab, 150).tolist()
    seq = rng.integers(0, n_seq, 150).tolist()
    assert decode_both(ctx, ref, toks, seq_id=seq, logits=[0] * 149 + [1], tol=tol) == 0
    for s, p0, p1 in ((1, 3, 20), (2, -1, 9), (0, 30, -1)):
        assert ctx.seq_rm(s, p0, p1) and ref.seq_rm(s, p0, p1)
    same_tables(ctx, ref)
    before = {(il, st): read_kv(ctx, il, st, ctx.n_cells)
              for il in (0, shape.n_layer - 1) for st in range(ref.n_stream)}
    moved = ctx.defrag()
    assert moved == ref.defrag() and moved > 0
    same_tables(ctx, ref)
    for (il, st), (k0, v0) in before.items():
        src = ref.last_defrag_src[st]
        k, v = read_kv(ctx, il, st, ctx.n_cells)
        assert np.array_equal(k[:src.size], k0[src]) and np.array_equal(v[:src.size], v0[src])
    assert ctx.defrag() == ref.defrag() == 0
    nxt = rng.integers(0, shape.n_vocab, n_seq).tolist()
    assert decode_both(ctx, ref, nxt, seq_id=list(range(n_seq)), logits=[1] * n_seq, tol=tol) == 0
    # seq_keep, then the kept sequence continues
    assert ctx.seq_keep(1) and ref.seq_keep(1)
    same_tables(ctx, ref)
    assert decode_both(ctx, ref, [5, 6], seq_id=[1, 1], logits=[1, 1], tol=tol) == 0


def test_full_cache_returns_1_and_changes_nothing(tiny):
    """A batch with no room in a fragmented cache returns 1 and leaves the
    cache as it was: cell tables, K/V rows and the logits of a following
    decode equal those of the oracle, which never ran the failed batch."""
    shape = tiny[0]
    ctx, ref = make(tiny, n_ctx=256, n_batch=256, n_ubatch=64, n_seq_max=2, kv_unified=True,
                    type_k="f16", type_v="f16")
    rng = np.random.default_rng(10)
    toks = rng.integers(0, shape.n_vocab, 200).tolist()
    assert decode_both(ctx, ref, toks, seq_id=[0, 1] * 100, logits=[0] * 199 + [1]) == 0
    # sequence 1 keeps positions < 50: the free cells are scattered
    assert ctx.seq_rm(1, 50, -1) and ref.seq_rm(1, 50, -1)
    before = ctx.cells(0)
    k_before = ctx.kv_read(0, 0, 0, 0, 256)
    assert ctx.decode([3] * 120, seq_id=[0] * 120) == 1
    assert ref.decode(Batch([3] * 120, seq_id=[0] * 120)) == 1
    assert all(np.array_equal(a, b) for a, b in zip(before, ctx.cells(0)))
    assert np.array_equal(k_before, ctx.kv_read(0, 0, 0, 0, 256))
    same_tables(ctx, ref)
    assert decode_both(ctx, ref, [4] * 6, seq_id=[0, 1] * 3, logits=[1] * 6) == 0


def test_defrag_at_large_cell_indices(tiny):
    """Two streams of 32768 cells: rows filled through kv_fill, holes cut
    with seq_rm, defrag moves rows from indices near the end."""
    shape = tiny[0]
    from llama_decode_ubatch_amd import Context
    ctx = Context(tiny[1], n_ctx=2 * 32768, n_batch=256, n_ubatch=64, n_seq_max=2, type_k="f16", type_v="f16")
    rng = np.random.default_rng(11)
    ne, n = shape.n_embd_kv, 32000
    K = [rng.standard_normal((n, ne)).astype(np.float16) for _ in range(shape.n_layer)]
    V = [rng.standard_normal((n, ne)).astype(np.float16) for _ in range(shape.n_layer)]
    for s in (0, 1):
        assert ctx.kv_fill(s, n, [k.view(np.uint16) for k in K], [v.view(np.uint16) for v in V], "f16") == 0
    assert ctx.seq_rm(1, 100, 31000)
    moved = ctx.defrag()
    assert moved == 1000
    pos, has = ctx.cells(1)
    assert pos[:1100].tolist() == list(range(100)) + list(range(31000, 32000)) and (pos[1100:] == -1).all()
    keep = np.r_[0:100, 31000:32000]
    for il in (0, shape.n_layer - 1):
        assert np.array_equal(ctx.kv_read(il, 1, 0, 0, 1100), K[il][keep].astype(np.float32))
        assert np.array_equal(ctx.kv_read(il, 1, 1, 0, 1100), V[il][keep].astype(np.float32))
        assert np.array_equal(ctx.kv_read(il, 0, 0, 31990, 10), K[il][31990:].astype(np.float32))
