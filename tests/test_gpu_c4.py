"""Attention-bound decode at full size (config 4): 16 sequences whose KV
streams are pre-filled through ubd_kv_fill with 32 704 positions of seeded
N(0,1) values, decoded one token per sequence per step (n_ctx 32 768 per
sequence).  Sampled checks: the stored KV equals the generator's values;
a sampled sequence's layer output equals the oracle's layer run from the
GPU's residual and the GPU's KV prefix; the logits of sampled sequences
equal the oracle head on the GPU's final residual; greedy ids match."""
import numpy as np
import pytest

from oracle import OracleModel, OracleContext
from workloads import WORKLOADS, gen_tensor, gen_tensor_rows, prompt_tokens, kv_prefill_block
from tests.helpers import oracle_layer_check

pytestmark = pytest.mark.gpu
TOL = 3e-2


def rel(a, b):
    return float(np.abs(np.asarray(a, np.float64) - b).max() / np.abs(b).max())


def fill_all(torch, ctx, w):
    from workloads import device as wdev
    P, L = w.kv_prefill, w.model.n_layer
    for s in range(w.n_seqs):
        K = [wdev.fill_kv_block(torch, w, s, il, 0, torch.empty((P, w.model.n_embd_kv), dtype=torch.int16,
                                                                  device="cuda:0")) for il in range(L)]
        V = [wdev.fill_kv_block(torch, w, s, il, 1, torch.empty((P, w.model.n_embd_kv), dtype=torch.int16,
                                                                  device="cuda:0")) for il in range(L)]
        torch.cuda.synchronize()
        assert ctx.kv_fill(s, P, K, V, "f16") == 0
        del K, V
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_config4_long_context_decode():
    import torch
    from llama_decode_ubatch_amd import Model, Context
    from workloads import device as wdev
    w = WORKLOADS[4]
    tens = wdev.model_tensors(torch, w.model, "cuda:0")
    torch.cuda.synchronize()
    model = Model(w.model, tens, device=0)
    del tens
    torch.cuda.empty_cache()
    ctx = Context(model, n_ctx=w.n_ctx, n_batch=w.n_batch, n_ubatch=w.n_ubatch, n_seq_max=w.n_seq_max,
                  type_k=w.type_k, type_v=w.type_v, kv_unified=w.kv_unified)
    print("config 4: filling 16 x 32704 KV positions", flush=True)
    fill_all(torch, ctx, w)
    P = w.kv_prefill
    for s in (0, 15):
        assert ctx.seq_pos_max(s) == P - 1
    # the cache holds exactly the generator's values (K rows and transposed V)
    np.testing.assert_array_equal(ctx.kv_read(7, 9, 0, 1000, 40),
                                  kv_prefill_block(w, 9, 7, 0, 1000, 40).view(np.float16).astype(np.float32))
    np.testing.assert_array_equal(ctx.kv_read(30, 3, 1, P - 40, 40),
                                  kv_prefill_block(w, 3, 30, 1, P - 40, 40).view(np.float16).astype(np.float32))
    om = OracleModel(w.model, lambda n: gen_tensor(w.model, n), dtype=np.float32, cache=True,
                     rows_fn=lambda n, r: gen_tensor_rows(w.model, n, r))
    ctx.keep_residuals(True)
    toks = np.array([prompt_tokens(w, s, 1)[0] for s in range(w.n_seqs)])
    seqs = np.arange(w.n_seqs)
    for step, (s, il) in enumerate(((9, 0), (0, 31), (5, 12))):
        assert ctx.decode(toks, seq_id=seqs, logits=np.ones(w.n_seqs)) == 0
        assert np.array_equal(ctx.last_ubatch(16), seqs)
        x_in, x_out = ctx.residual(il, 16)[s], ctx.residual(il + 1, 16)[s]
        n = P + step
        K = ctx.kv_read(il, s, 0, 0, n).astype(np.float16)
        V = ctx.kv_read(il, s, 1, 0, n).astype(np.float16)
        y, _ = oracle_layer_check(om, w, il, x_in[None, :], [int(toks[s])], n, (K, V))
        err = rel(x_out[None, :], y)
        print(f"  step {step} seq {s} layer {il}: rel err {err:.2e}", flush=True)
        assert err < TOL
        z_all = ctx.logits()
        x_last = ctx.residual(w.model.n_layer, 16)
        for s2 in (s, 14):
            zr = OracleContext(om, 512).head(x_last[s2:s2 + 1].astype(np.float32))[0]
            assert rel(z_all[s2], zr) < TOL, s2
        ids = ctx.greedy_all()
        assert np.array_equal(ids, np.argmax(z_all, axis=1))
        toks = ids
    for s in (0, 15):
        assert ctx.seq_pos_max(s) == P + 2
