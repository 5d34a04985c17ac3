"""Pins for oracle/model.py: the invariants the method fixes (prefill ==
token-by-token decode, ubatch-split invariance, GQA == replicated heads,
unified == per-sequence streams, sequence isolation, rollback, RoPE shift
invariance) and a brute-force no-cache forward on tiny inputs (CPU only)."""
import math

import numpy as np
import pytest
from scipy.special import expit

from oracle import Batch
from tests.helpers import MICRO, micro_tensors, oracle_ctx, rand_tokens
from workloads import ModelShape

TENS = micro_tensors()


def _prefill_all(ctx, toks, **kw):
    assert ctx.decode(Batch(toks, logits=np.ones(len(toks), np.int8), **kw)) == 0
    return np.stack([ctx.logits_ith(i) for i in range(len(toks))])


def _one_by_one(ctx, toks):
    rows = []
    for t in toks:
        assert ctx.decode(Batch([t])) == 0
        rows.append(ctx.logits_ith(-1).copy())
    return np.stack(rows)


def test_prefill_equals_token_by_token_decode():
    toks = rand_tokens(23, MICRO.n_vocab, 0)
    a = _prefill_all(oracle_ctx(tensors=TENS), toks)
    b = _one_by_one(oracle_ctx(tensors=TENS), toks)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * np.abs(a).max())


@pytest.mark.parametrize("n_ubatch", [1, 7, 32, 128])
def test_ubatch_split_invariance(n_ubatch):
    toks = rand_tokens(40, MICRO.n_vocab, 1)
    ref_ctx = oracle_ctx(tensors=TENS, n_batch=256, n_ubatch=256)
    ref = _prefill_all(ref_ctx, toks)
    ctx = oracle_ctx(tensors=TENS, n_batch=256, n_ubatch=n_ubatch)
    out = _prefill_all(ctx, toks)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12 * np.abs(ref).max())
    assert np.array_equal(np.concatenate(ctx.last_plan.cells),
                          np.concatenate(ref_ctx.last_plan.cells))
    assert len(ctx.last_plan.ubatches) == math.ceil(40 / n_ubatch)


def _rope_complex(x, pos, base):
    z = x[..., 0::2] + 1j * x[..., 1::2]
    hd = x.shape[-1]
    th = base ** (-np.arange(hd // 2) * 2.0 / hd)
    w = z * np.exp(1j * pos[:, None, None] * th)
    out = np.empty_like(x)
    out[..., 0::2], out[..., 1::2] = w.real, w.imag
    return out


def _brute_forward(shape, tens, toks):
    """No cache, no cells: every token of one sequence attends to tokens
    0..t by explicit loops."""
    W = lambda n: tens[n]["data"].astype(np.float64)
    H, Hk, hd, eps = shape.n_head, shape.n_head_kv, shape.head_dim, shape.rms_eps
    T = len(toks)
    pos = np.arange(T)
    norm = lambda v, g: v / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps) * g
    x = W("token_embd.weight")[toks]
    for il in range(shape.n_layer):
        p = f"blk.{il}."
        xn = norm(x, W(p + "attn_norm.weight"))
        q = _rope_complex((xn @ W(p + "attn_q.weight").T).reshape(T, H, hd), pos, shape.rope_base)
        k = _rope_complex((xn @ W(p + "attn_k.weight").T).reshape(T, Hk, hd), pos, shape.rope_base)
        v = (xn @ W(p + "attn_v.weight").T).reshape(T, Hk, hd)
        # the cache stores K and V as f32 (type_k = type_v = f32)
        k = k.astype(np.float32).astype(np.float64)
        v = v.astype(np.float32).astype(np.float64)
        out = np.zeros((T, H, hd))
        for t in range(T):
            for h in range(H):
                kvh = h // (H // Hk)
                sc = [float(q[t, h] @ k[s, kvh]) / math.sqrt(hd) for s in range(t + 1)]
                mx = max(sc)
                e = [math.exp(v_ - mx) for v_ in sc]
                z = sum(e)
                for s in range(t + 1):
                    out[t, h] += e[s] / z * v[s, kvh]
        x = x + out.reshape(T, H * hd) @ W(p + "attn_output.weight").T
        xn = norm(x, W(p + "ffn_norm.weight"))
        g_ = xn @ W(p + "ffn_gate.weight").T
        x = x + (g_ * expit(g_) * (xn @ W(p + "ffn_up.weight").T)) @ W(p + "ffn_down.weight").T
    return norm(x, W("output_norm.weight")) @ W("output.weight").T


def test_bruteforce_no_cache_forward():
    toks = rand_tokens(9, MICRO.n_vocab, 2)
    a = _prefill_all(oracle_ctx(tensors=TENS, n_ubatch=4), toks)
    np.testing.assert_allclose(a, _brute_forward(MICRO, TENS, toks), rtol=0,
                               atol=1e-11 * np.abs(a).max())


def test_tied_output_uses_the_embedding_table():
    """A model without output.weight takes its logits from token_embd (the
    engine page's Step 6: the output tensor is optional and duplicates the
    embedding); the brute-force forward gets the table under both names."""
    tied = {k: v for k, v in TENS.items() if k != "output.weight"}
    both = dict(tied, **{"output.weight": TENS["token_embd.weight"]})
    toks = rand_tokens(9, MICRO.n_vocab, 12)
    ctx = oracle_ctx(tensors=tied, n_ubatch=4)
    assert ctx.model.tied
    a = _prefill_all(ctx, toks)
    np.testing.assert_allclose(a, _brute_forward(MICRO, both, toks), rtol=0,
                               atol=1e-11 * np.abs(a).max())
    # and the untied model differs, so the test sees which table was used
    assert np.abs(a - _prefill_all(oracle_ctx(tensors=TENS, n_ubatch=4), toks)).max() > 1e-3 * np.abs(a).max()


def test_gqa_equals_replicated_heads():
    mha = ModelShape("micro-mha", 10, n_layer=MICRO.n_layer, n_embd=MICRO.n_embd,
                     n_head=MICRO.n_head, n_head_kv=MICRO.n_head,
                     n_ff=MICRO.n_ff, n_vocab=MICRO.n_vocab, n_ctx_train=512,
                     rope_base=MICRO.rope_base)
    hd, g = MICRO.head_dim, MICRO.n_gqa
    t2 = dict(TENS)
    for il in range(MICRO.n_layer):
        for w in ("attn_k", "attn_v"):
            name = f"blk.{il}.{w}.weight"
            rows = TENS[name]["data"].reshape(MICRO.n_head_kv, hd, -1)
            t2[name] = {"type": "f32", "data": np.repeat(rows, g, axis=0).reshape(-1, MICRO.n_embd)}
    toks = rand_tokens(12, MICRO.n_vocab, 3)
    a = _prefill_all(oracle_ctx(tensors=TENS), toks)
    b = _prefill_all(oracle_ctx(shape=mha, tensors=t2), toks)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-12 * np.abs(a).max())


def _multi_seq_batch(seed):
    rng = np.random.default_rng(seed)
    seq = rng.permutation(np.repeat(np.arange(3), [5, 7, 4]))
    toks = rng.integers(0, MICRO.n_vocab, seq.size)
    return toks, seq


def test_unified_equals_per_sequence_streams():
    toks, seq = _multi_seq_batch(4)
    outs = []
    for unified in (True, False):
        ctx = oracle_ctx(tensors=TENS, n_ctx=768, n_seq_max=3, kv_unified=unified, n_ubatch=5)
        outs.append(_prefill_all(ctx, toks, seq_id=seq))
        assert ctx.decode(Batch([1, 2, 3], seq_id=[2, 0, 1], logits=[1, 1, 1])) == 0
        outs.append(np.stack([ctx.logits_ith(i) for i in range(3)]))
    np.testing.assert_allclose(outs[0], outs[2], rtol=0, atol=1e-12)
    np.testing.assert_allclose(outs[1], outs[3], rtol=0, atol=1e-12)


def test_sequence_isolation():
    toks, seq = _multi_seq_batch(5)
    ctx = oracle_ctx(tensors=TENS, n_ctx=768, n_seq_max=3, kv_unified=True)
    mixed = _prefill_all(ctx, toks, seq_id=seq)
    for s in range(3):
        alone = _prefill_all(oracle_ctx(tensors=TENS, n_ctx=768, n_seq_max=3),
                             toks[seq == s], seq_id=np.full((seq == s).sum(), s))
        np.testing.assert_allclose(mixed[seq == s], alone, rtol=0, atol=1e-12)


def test_rope_shift_invariance_of_whole_model():
    toks = rand_tokens(10, MICRO.n_vocab, 6)
    a = _prefill_all(oracle_ctx(tensors=TENS), toks)
    b = _prefill_all(oracle_ctx(tensors=TENS), toks, pos=np.arange(1000, 1010))
    # K/V are stored as f32, so rotated keys round differently: f32-level error
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-6 * np.abs(a).max())


@pytest.mark.parametrize("k", [0, 1, 2])
def test_abort_rolls_back_to_completed_ubatches(k):
    toks = rand_tokens(12, MICRO.n_vocab, 7)
    ctx = oracle_ctx(tensors=TENS, n_ubatch=4)
    assert ctx.decode(Batch(toks), abort_at=k) == 2
    assert ctx.seq_pos_max(0) == 4 * k - 1
    ref = oracle_ctx(tensors=TENS, n_ubatch=4)
    if k:
        assert ref.decode(Batch(toks[:4 * k])) == 0
    assert np.array_equal(ctx.mem.pos, ref.mem.pos)
    # continuing after the rollback gives the same logits as the clean context
    rest = toks[4 * k:]
    assert ctx.decode(Batch(rest)) == 0 and ref.decode(Batch(rest)) == 0
    np.testing.assert_array_equal(ctx.logits_ith(-1), ref.logits_ith(-1))
    assert ctx.decode(Batch(toks[:2]), fail_at=0) == -3
    assert ctx.seq_pos_max(0) == 11


def test_no_slot_leaves_state_unchanged():
    ctx = oracle_ctx(tensors=TENS, n_ctx=256)
    assert ctx.decode(Batch(rand_tokens(250, MICRO.n_vocab, 8))) == 0
    pos = ctx.mem.pos.copy()
    assert ctx.decode(Batch(rand_tokens(7, MICRO.n_vocab, 9))) == 1
    assert np.array_equal(ctx.mem.pos, pos)
    assert ctx.decode(Batch(rand_tokens(6, MICRO.n_vocab, 9))) == 0


def test_logits_ith_indexing_and_greedy():
    ctx = oracle_ctx(tensors=TENS)
    toks = rand_tokens(5, MICRO.n_vocab, 10)
    assert ctx.decode(Batch(toks, logits=[0, 1, 0, 1, 1])) == 0
    assert ctx.logits_ith(0) is None and ctx.logits_ith(2) is None
    np.testing.assert_array_equal(ctx.logits_ith(-1), ctx.logits_ith(4))
    np.testing.assert_array_equal(ctx.logits_ith(-3), ctx.logits_ith(1))
    assert ctx.logits_ith(-4) is None
    z = ctx.logits_ith(3)
    assert ctx.greedy(3) == int(np.argmax(z))
    ctx.logits[ctx.out_row[3], :] = 0.0          # all tied -> lowest id
    assert ctx.greedy(3) == 0


def test_kv_f16_storage_changes_only_by_rounding():
    toks = rand_tokens(16, MICRO.n_vocab, 11)
    a = _prefill_all(oracle_ctx(tensors=TENS), toks)
    b = _prefill_all(oracle_ctx(tensors=TENS, type_k="f16", type_v="f16"), toks)
    err = np.abs(a - b).max() / np.abs(a).max()
    assert 0 < err < 1e-2
