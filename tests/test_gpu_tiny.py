"""GPU parity on the tiny f32 model (configs 1 and 2) through the C ABI:
logits within 1e-4 of the logit max-norm, greedy ids and KV cells exact,
plus edge cases (split invariance, return codes, rollback, unified KV,
KV fill/read, residual dumps)."""
import numpy as np
import pytest

from oracle import OracleModel, OracleContext, Batch
from workloads import WORKLOADS, gen_tensor, tensor_specs, prompt_tokens

pytestmark = pytest.mark.gpu
TOL = 1e-4          # fp32 configs: max |dz| <= 1e-4 * max |z_oracle|


def rel_err(z, zr):
    return float(np.abs(np.asarray(z, np.float64) - zr).max() / np.abs(zr).max())


@pytest.fixture(scope="module")
def tiny():
    import torch
    from llama_decode_ubatch_amd import Model
    assert torch.cuda.is_available()
    shape = WORKLOADS[1].model
    tens = {s.name: gen_tensor(shape, s) for s in tensor_specs(shape)}
    model = Model(shape, tens, device=0)
    om = OracleModel(shape, tens, dtype=np.float64)
    return shape, tens, model, om


def make(tiny, **kw):
    from llama_decode_ubatch_amd import Context
    shape, tens, model, om = tiny
    ctx = Context(model, **kw)
    ref = OracleContext(om, **kw)
    return ctx, ref


def test_config1_prefill_then_greedy(tiny):
    w = WORKLOADS[1]
    ctx, ref = make(tiny, n_ctx=w.n_ctx, n_batch=w.n_batch, n_ubatch=w.n_ubatch, n_seq_max=1,
                    type_k=w.type_k, type_v=w.type_v)
    prompt = prompt_tokens(w, 0)
    print(f"config 1: prompt {prompt.size} tokens", flush=True)
    assert ctx.decode(prompt) == 0 and ref.decode(Batch(prompt)) == 0
    assert np.array_equal(ctx.kv_cells(prompt.size), np.concatenate(ref.last_plan.cells))
    for step in range(w.n_decode + 1):
        z, zr = ctx.logits_ith(-1), ref.logits_ith(-1)
        assert rel_err(z, zr) < TOL, step
        tok = ctx.greedy(-1)
        assert tok == ref.greedy(-1), step
        if step == w.n_decode:
            break
        assert ctx.decode([tok]) == 0 and ref.decode(Batch([tok])) == 0
        assert ctx.kv_cells(1)[0] == ref.last_plan.cells[0][0]
    assert ctx.seq_pos_max(0) == prompt.size + w.n_decode - 1


def test_config2_eight_sequences(tiny):
    w = WORKLOADS[2]
    ctx, ref = make(tiny, n_ctx=w.n_ctx, n_batch=w.n_batch, n_ubatch=w.n_ubatch, n_seq_max=w.n_seq_max,
                    type_k=w.type_k, type_v=w.type_v)
    toks = np.concatenate([prompt_tokens(w, s) for s in range(w.n_seqs)])
    seq = np.repeat(np.arange(w.n_seqs), w.n_prompt)
    out = np.zeros(toks.size, np.int8)
    out[w.n_prompt - 1::w.n_prompt] = 1
    print(f"config 2: batch of {toks.size} tokens", flush=True)
    assert ctx.decode(toks, seq_id=seq, logits=out) == 0
    assert ref.decode(Batch(toks, seq_id=seq, logits=out)) == 0
    assert np.array_equal(ctx.kv_cells(toks.size),
                          np.concatenate([c for c in ref.last_plan.cells])[np.argsort(
                              np.concatenate([u.idx for u in ref.last_plan.ubatches]))])
    ids = ctx.greedy_all()
    for step in range(w.n_decode + 1):
        z, zr = ctx.logits(), ref.logits
        assert z.shape == zr.shape
        assert rel_err(z, zr) < TOL, step
        ids_ref = np.array([ref.greedy(int(i)) for i in np.flatnonzero(ref.out_row >= 0)])
        ids = ctx.greedy_all()
        assert np.array_equal(ids, ids_ref), step
        if step == w.n_decode:
            break
        assert ctx.decode(ids, seq_id=np.arange(w.n_seqs), logits=np.ones(w.n_seqs)) == 0
        assert ref.decode(Batch(ids, seq_id=np.arange(w.n_seqs), logits=np.ones(w.n_seqs))) == 0
    for s in range(w.n_seqs):
        assert ctx.seq_pos_max(s) == w.n_prompt + w.n_decode - 1


@pytest.mark.parametrize("n_ubatch", [1, 7, 16, 33])
def test_all_logits_split_invariance(tiny, n_ubatch):
    toks = prompt_tokens(WORKLOADS[1], 1, 40)
    ctx, ref = make(tiny, n_ctx=256, n_batch=64, n_ubatch=n_ubatch, type_k="f32", type_v="f32")
    flags = np.ones(toks.size, np.int8)
    assert ctx.decode(toks, logits=flags) == 0 and ref.decode(Batch(toks, logits=flags)) == 0
    assert rel_err(ctx.logits(), ref.logits) < TOL
    assert np.array_equal(ctx.greedy_all(), np.argmax(ref.logits, axis=1))


def test_unified_interleaved_sequences(tiny):
    rng = np.random.default_rng(3)
    seq = rng.permutation(np.repeat(np.arange(3), [9, 13, 6]))
    toks = rng.integers(0, WORKLOADS[1].model.n_vocab, seq.size)
    for unified in (True, False):
        ctx, ref = make(tiny, n_ctx=768, n_batch=64, n_ubatch=10, n_seq_max=3, kv_unified=unified,
                        type_k="f16", type_v="f16")
        flags = np.ones(seq.size, np.int8)
        assert ctx.decode(toks, seq_id=seq, logits=flags) == 0
        assert ref.decode(Batch(toks, seq_id=seq, logits=flags)) == 0
        assert rel_err(ctx.logits(), ref.logits) < TOL
        nxt = [ctx.greedy(int(np.flatnonzero(seq == s)[-1])) for s in range(3)]
        assert ctx.decode(nxt, seq_id=[0, 1, 2], logits=[1, 1, 1]) == 0
        assert ref.decode(Batch(nxt, seq_id=[0, 1, 2], logits=[1, 1, 1])) == 0
        assert rel_err(ctx.logits(), ref.logits) < TOL


@pytest.mark.parametrize("kv, tol", [("f16", TOL), ("q8_0", 2e-3)])
def test_ragged_sequences_split_attention(tiny, kv, tol):
    """Three sequences of 20, 150 and 300 cells decode one token each in one
    ubatch: the split attention launches chunks for the longest scan, so with
    per-sequence KV streams the shorter sequences' tiles carry empty chunks
    (m = -inf, l = 0) into the combine; the unified stream scans all cells
    with masks.  f16 and q8_0 caches (the q8_0 tolerance is that of the other
    q8_0 cache tests)."""
    rng = np.random.default_rng(11)
    V = WORKLOADS[1].model.n_vocab
    lens = [20, 150, 300]
    for unified in (True, False):
        ctx, ref = make(tiny, n_ctx=1536, n_batch=512, n_ubatch=512, n_seq_max=3, kv_unified=unified,
                        type_k=kv, type_v=kv)
        for s, n in enumerate(lens):
            toks = rng.integers(0, V, n)
            assert ctx.decode(toks, seq_id=np.full(n, s)) == 0
            assert ref.decode(Batch(toks, seq_id=np.full(n, s))) == 0
        nxt = rng.integers(0, V, 3)
        assert ctx.decode(nxt, seq_id=[0, 1, 2], logits=[1, 1, 1]) == 0
        assert ref.decode(Batch(nxt, seq_id=[0, 1, 2], logits=[1, 1, 1])) == 0
        assert rel_err(ctx.logits(), ref.logits) < tol
        if kv == "f16":
            assert [ctx.greedy(i) for i in range(3)] == [int(np.argmax(ref.logits[i])) for i in range(3)]


def test_long_scan_many_chunks(tiny):
    """One sequence of 4200 cells, then a one-token decode: the split
    attention cuts the scan into 66 chunks of 64 cells, so the combine pass
    takes them in two groups (64, then 2)."""
    rng = np.random.default_rng(12)
    V = WORKLOADS[1].model.n_vocab
    ctx, ref = make(tiny, n_ctx=4608, n_batch=512, n_ubatch=512, type_k="f16", type_v="f16")
    toks = rng.integers(0, V, 4200)
    for i in range(0, toks.size, 512):
        assert ctx.decode(toks[i:i + 512]) == 0
        assert ref.decode(Batch(toks[i:i + 512])) == 0
    nxt = [int(rng.integers(0, V))]
    assert ctx.decode(nxt, logits=[1]) == 0
    assert ref.decode(Batch(nxt, logits=[1])) == 0
    assert rel_err(ctx.logits(), ref.logits) < TOL
    assert ctx.greedy(0) == int(np.argmax(ref.logits[0]))


@pytest.mark.parametrize("kv", ["f16", "q8_0"])
def test_non_temporal_kv_loads_give_the_same_logits(tiny, kv):
    """Split attention streams K/V with non-temporal loads only when a launch
    reads at least attn_nt_mb MB; forcing that path (0) on ragged sequences
    reads the same values, so the logits equal the cached-load run bit for
    bit, and both are within the oracle's tolerance."""
    from llama_decode_ubatch_amd.binding import set_tuning
    rng = np.random.default_rng(13)
    V = WORKLOADS[1].model.n_vocab
    lens = [40, 333, 700]
    toks = [rng.integers(0, V, n) for n in lens]
    nxt = rng.integers(0, V, 3)
    out = []
    for nt in (32, 0):
        set_tuning("attn_nt_mb", nt)
        try:
            ctx, ref = make(tiny, n_ctx=3072, n_batch=1024, n_ubatch=1024, n_seq_max=3, type_k=kv, type_v=kv)
            for s, t in enumerate(toks):
                assert ctx.decode(t, seq_id=np.full(t.size, s)) == 0
            assert ctx.decode(nxt, seq_id=[0, 1, 2], logits=[1, 1, 1]) == 0
            out.append(ctx.logits())
        finally:
            set_tuning("attn_nt_mb", 32)
    print(f"{kv}: max |dz| between the load paths {float(np.abs(out[0] - out[1]).max()):.1e}", flush=True)
    assert np.array_equal(out[0], out[1])
    for s, t in enumerate(toks):
        assert ref.decode(Batch(t, seq_id=np.full(t.size, s))) == 0
    assert ref.decode(Batch(nxt, seq_id=[0, 1, 2], logits=[1, 1, 1])) == 0
    assert rel_err(out[1], ref.logits) < (TOL if kv == "f16" else 2e-3)


def test_return_codes_abort_and_rollback(tiny):
    from llama_decode_ubatch_amd import Context
    shape, tens, model, om = tiny
    calls = {"n": 0, "stop_at": -1}

    def abort():
        calls["n"] += 1
        return calls["n"] - 1 == calls["stop_at"]

    ctx = Context(model, n_ctx=256, n_batch=128, n_ubatch=8, type_k="f32", type_v="f32",
                  abort_callback=abort)
    ref = OracleContext(om, n_ctx=256, n_batch=128, n_ubatch=8, type_k="f32", type_v="f32")
    toks = prompt_tokens(WORKLOADS[1], 2, 20)
    assert ctx.decode(np.zeros(0, int)) == -1
    assert ctx.decode([shape.n_vocab]) == -1
    assert ctx.decode([1], seq_id=[1]) == -1
    assert ctx.decode(np.ones(129, int)) == -1
    calls["n"], calls["stop_at"] = 0, 2          # abort at the third ubatch
    assert ctx.decode(toks) == 2
    assert ctx.seq_pos_max(0) == 15
    assert ref.decode(Batch(toks[:16])) == 0
    calls["stop_at"] = -1
    assert ctx.decode(toks[16:]) == 0 and ref.decode(Batch(toks[16:])) == 0
    assert rel_err(ctx.logits_ith(-1), ref.logits_ith(-1)) < TOL
    # seq_rm the tail, then decode it again
    assert ctx.seq_rm(0, 10, -1) and ref.seq_rm(0, 10, -1)
    assert ctx.decode(toks[10:]) == 0 and ref.decode(Batch(toks[10:])) == 0
    assert rel_err(ctx.logits_ith(-1), ref.logits_ith(-1)) < TOL
    # fill the cache: no slot -> 1, nothing changes
    big = prompt_tokens(WORKLOADS[1], 3, 128)
    assert ctx.decode(big) == 0 and ref.decode(Batch(big)) == 0
    big2 = prompt_tokens(WORKLOADS[1], 4, 120)
    assert ctx.decode(big2) == 1 and ref.decode(Batch(big2)) == 1
    assert ctx.seq_pos_max(0) == ref.seq_pos_max(0)
    assert ctx.decode(big2[:8]) == 0 and ref.decode(Batch(big2[:8])) == 0
    assert rel_err(ctx.logits_ith(-1), ref.logits_ith(-1)) < TOL


def test_kv_fill_and_read(tiny):
    shape = tiny[0]
    rng = np.random.default_rng(5)
    n = 70
    k = [rng.standard_normal((n, shape.n_embd_kv)).astype(np.float16) for _ in range(shape.n_layer)]
    v = [rng.standard_normal((n, shape.n_embd_kv)).astype(np.float16) for _ in range(shape.n_layer)]
    ctx, ref = make(tiny, n_ctx=512, n_batch=64, n_ubatch=32, n_seq_max=2, type_k="f16", type_v="f16")
    assert ctx.kv_fill(1, n, [a.view(np.uint16) for a in k], [a.view(np.uint16) for a in v], "f16") == 0
    assert ref.kv_fill(1, n, k, v)
    assert ctx.seq_pos_max(1) == n - 1
    np.testing.assert_array_equal(ctx.kv_read(2, 1, 0, 0, n), k[2].astype(np.float32))
    np.testing.assert_array_equal(ctx.kv_read(3, 1, 1, 0, n), v[3].astype(np.float32))
    toks = prompt_tokens(WORKLOADS[1], 5, 5)
    flags = np.ones(5, np.int8)
    assert ctx.decode(toks, seq_id=[1] * 5, logits=flags) == 0
    assert ref.decode(Batch(toks, seq_id=[1] * 5, logits=flags)) == 0
    assert rel_err(ctx.logits(), ref.logits) < TOL
    # the cache holds exactly what the oracle stored for the new tokens
    Kr, _ = ref.kv(0, 1)
    np.testing.assert_allclose(ctx.kv_read(0, 1, 0, n, 5), Kr[n:n + 5].astype(np.float32), rtol=1e-3, atol=1e-3)


def test_residual_stream_per_layer(tiny):
    shape = tiny[0]
    ctx, ref = make(tiny, n_ctx=256, n_batch=64, n_ubatch=64, type_k="f32", type_v="f32")
    assert ctx.keep_residuals(True) == 0
    ref.record = {}
    toks = prompt_tokens(WORKLOADS[1], 6, 12)
    assert ctx.decode(toks) == 0 and ref.decode(Batch(toks)) == 0
    for il in range(shape.n_layer + 1):
        xg, xr = ctx.residual(il, 64), ref.record["x"][il]
        assert float(np.abs(xg - xr).max() / np.abs(xr).max()) < 1e-5, il
