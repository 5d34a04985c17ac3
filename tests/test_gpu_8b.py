"""8B-shaped parity at full size, in the launch configuration bench.py
times (512-token prefill as one ubatch, then single-token decode), on
sampled outputs the oracle computes one by one: the oracle re-runs sampled
layers from the GPU's own input to that layer and the output head from the
GPU's final residual.  Tolerance (bf16 / int8 configs): max |error| within
3e-2 of the max-norm of the oracle's output; the prefill layers, whose
products take the activations as hi + lo planes, within 2e-3."""
import numpy as np
import pytest

from oracle import OracleModel, OracleContext, Batch
from workloads import WORKLOADS, gen_tensor, gen_tensor_rows, prompt_tokens
from tests.helpers import oracle_layer_check

pytestmark = pytest.mark.gpu
TOL = 3e-2
TOL_PREFILL_LAYER = 2e-3
PREFILL_LAYERS = tuple(range(0, 32, 4)) + (1, 31)


def rel(a, b):
    return float(np.abs(np.asarray(a, np.float64) - b).max() / np.abs(b).max())


def build(cfg):
    import torch
    from llama_decode_ubatch_amd import Model
    from workloads import device as wdev
    w = WORKLOADS[cfg]
    tens = wdev.model_tensors(torch, w.model, "cuda:0")
    torch.cuda.synchronize()
    model = Model(w.model, tens, device=0)
    del tens
    torch.cuda.empty_cache()
    om = OracleModel(w.model, lambda n: gen_tensor(w.model, n), dtype=np.float32, cache=True,
                     rows_fn=lambda n, r: gen_tensor_rows(w.model, n, r))
    return w, model, om


def oracle_layer(om, w, il, x_in, tokens, pos0, kv_prefix=None):
    return oracle_layer_check(om, w, il, x_in, tokens, pos0, kv_prefix)


@pytest.mark.parametrize("cfg", [3, 5])
def test_prefill_and_decode_sampled_layers(cfg):
    from llama_decode_ubatch_amd import Context
    w, model, om = build(cfg)
    ctx = Context(model, n_ctx=w.n_ctx, n_batch=w.n_batch, n_ubatch=w.n_ubatch, type_k=w.type_k,
                  type_v=w.type_v)
    assert ctx.keep_residuals(True) == 0
    prompt = prompt_tokens(w, 0)
    T = prompt.size
    print(f"config {cfg}: prefill {T} tokens", flush=True)
    assert ctx.decode(prompt) == 0
    for il in PREFILL_LAYERS:
        x_in, x_out = ctx.residual(il, T), ctx.residual(il + 1, T)
        y, ref = oracle_layer(om, w, il, x_in, prompt, 0)
        err = rel(x_out, y)
        print(f"  prefill layer {il}: rel err {err:.2e}", flush=True)
        assert err < TOL_PREFILL_LAYER, il
        # the K/V this layer appended, as stored (f16)
        Kr, Vr = ref.kv(il, 0)
        assert rel(ctx.kv_read(il, 0, 0, 0, T), Kr[:T].astype(np.float32)) < TOL
        assert rel(ctx.kv_read(il, 0, 1, 0, T), Vr[:T].astype(np.float32)) < TOL
    x_last = ctx.residual(w.model.n_layer, T)[-1:]
    zr = OracleContext(om, w.n_ctx).head(x_last.astype(np.float32))[0]
    z = ctx.logits_ith(-1)
    print(f"  prefill logits: rel err {rel(z, zr):.2e}", flush=True)
    assert rel(z, zr) < TOL and int(np.argmax(z)) == int(np.argmax(zr))
    tok = ctx.greedy(-1)
    assert tok == int(np.argmax(z))
    # three decode steps, each checked at a sampled layer with the GPU's KV prefix
    for step, il in enumerate((0, 31, 5)):
        assert ctx.decode([tok]) == 0
        p = T + step
        x_in, x_out = ctx.residual(il, 1), ctx.residual(il + 1, 1)
        K = ctx.kv_read(il, 0, 0, 0, p).astype(np.float16)
        V = ctx.kv_read(il, 0, 1, 0, p).astype(np.float16)
        y, _ = oracle_layer(om, w, il, x_in, np.array([tok]), p, (K, V))
        err = rel(x_out, y)
        print(f"  decode step {step} layer {il}: rel err {err:.2e}", flush=True)
        assert err < TOL
        x_last = ctx.residual(w.model.n_layer, 1)
        zr = OracleContext(om, w.n_ctx).head(x_last.astype(np.float32))[0]
        z = ctx.logits_ith(-1)
        assert rel(z, zr) < TOL
        tok = ctx.greedy(-1)
        assert tok == int(np.argmax(z))
    # one-token products with the activation loads issued after the weight
    # loads: the same arithmetic, so the same logits bit for bit (two
    # one-token ubatches: no split-k product, whose atomic partial sums
    # make the order of additions vary from run to run)
    from llama_decode_ubatch_amd.binding import set_tuning
    z_early = []
    for early in (1, 0):
        set_tuning("ldsx_early", early)
        try:
            c2 = Context(model, n_ctx=w.n_ctx, n_batch=w.n_batch, n_ubatch=w.n_ubatch, type_k=w.type_k,
                         type_v=w.type_v)
            assert c2.decode(prompt[:1]) == 0 and c2.decode([tok]) == 0
            z_early.append(c2.logits_ith(-1).copy())
            c2.free()
        finally:
            set_tuning("ldsx_early", 1)
    assert np.array_equal(z_early[0], z_early[1])
    ctx.free()
    model.free()


@pytest.mark.parametrize("cfg", [3, 5])
def test_few_token_ubatch_sampled_layers(cfg):
    """A 7-token prompt: below the GEMM threshold and above the fused-norm
    one, so every product runs as a few-token product with several row
    blocks per work-group (gate|up, logits) or k split over work-groups
    (O, down), all 7 logits rows requested."""
    from llama_decode_ubatch_amd import Context
    w, model, om = build(cfg)
    ctx = Context(model, n_ctx=w.n_ctx, n_batch=w.n_batch, n_ubatch=w.n_ubatch, type_k=w.type_k,
                  type_v=w.type_v)
    assert ctx.keep_residuals(True) == 0
    prompt = prompt_tokens(w, 0)[:7]
    T = prompt.size
    assert ctx.decode(prompt, logits=np.ones(T)) == 0
    for il in (0, 31):
        x_in, x_out = ctx.residual(il, T), ctx.residual(il + 1, T)
        y, _ = oracle_layer(om, w, il, x_in, prompt, 0)
        err = rel(x_out, y)
        print(f"  {T}-token ubatch layer {il}: rel err {err:.2e}", flush=True)
        assert err < TOL, il
    z = ctx.logits()
    zr = OracleContext(om, 512).head(ctx.residual(w.model.n_layer, T).astype(np.float32))
    err = rel(z, zr)
    print(f"  {T}-token ubatch logits: rel err {err:.2e}", flush=True)
    assert err < TOL
    om.drop_cache()
