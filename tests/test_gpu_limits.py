"""Decode products at the edges of their fast paths, against the oracle.

* A model 9216 values wide: one token's normalised row (36 KB) fits the
  LDS stage of the one-token products, two or three tokens' rows (72 KB,
  108 KB) do not, so those ubatches normalise their rows on the fly in the
  few-token products.  Every logits row is compared with the float64 oracle
  (f32 weights, 1e-4 of the logit max-norm).
* q8_0 decode products stage their activations as f16 hi + lo planes,
  which end at 65504.  Norm gains of 1e5 on a few channels (attention norm
  of layer 0, FFN norm of layer 1, output norm) make the inputs of the QKV,
  gate|up and logits products exceed that, and the SwiGLU output entering
  the FFN down product exceeds it by orders of magnitude.  The oracle's own
  activations confirm the planted values pass 65504; the logits must still
  match the oracle within the q8_0 tolerance (2e-3 of the max-norm).
"""
import numpy as np
import pytest

from oracle import Batch
from oracle import numerics as nm
from workloads import ModelShape, gen_tensor, tensor_specs
from tests.helpers import oracle_ctx, rand_tokens

WIDE = ModelShape("wide-f32", 15, n_layer=1, n_embd=9216, n_head=72, n_head_kv=9, n_ff=64,
                  n_vocab=512, n_ctx_train=512, rope_base=10000.0, wtype="f32")
BIG = ModelShape("small-q8-big", 14, n_layer=2, n_embd=256, n_head=8, n_head_kv=2, n_ff=1408,
                 n_vocab=1024, n_ctx_train=2048, rope_base=10000.0, wtype="q8_0")
PLANTED = ("blk.0.attn_norm.weight", "blk.1.ffn_norm.weight", "output_norm.weight")
F16_MAX = 65504.0


def rel_err(z, zr):
    return float(np.abs(np.asarray(z, np.float64) - zr).max() / np.abs(zr).max())


def run_both(model, shape, tens, tokens, steps, type_kv, tol, label):
    """Prefill `tokens` (every row flagged), then `steps` one-token decodes
    of the oracle's greedy picks; all logits against the oracle."""
    from llama_decode_ubatch_amd import Context
    ctx = Context(model, n_ctx=512, n_batch=512, n_ubatch=512, n_seq_max=1, type_k=type_kv, type_v=type_kv)
    ref = oracle_ctx(shape, tens, np.float64, n_ctx=512, n_batch=512, n_ubatch=512, type_k=type_kv,
                     type_v=type_kv)
    n = len(tokens)
    assert ctx.decode(tokens, logits=np.ones(n)) == 0
    assert ref.decode(Batch(tokens, logits=[1] * n)) == 0
    zr = np.stack([ref.logits_ith(i) for i in range(n)])
    err = rel_err(ctx.logits(), zr)
    print(f"{label} T={n}: logits rel err {err:.2e}", flush=True)
    assert err < tol
    for step in range(steps):
        tok = ref.greedy(-1)
        assert ctx.decode([tok]) == 0 and ref.decode(Batch([tok])) == 0
        err = rel_err(ctx.logits_ith(-1), ref.logits_ith(-1))
        print(f"{label} T={n} step {step}: logits rel err {err:.2e}", flush=True)
        assert err < tol
    ctx.free()


@pytest.fixture(scope="module")
def wide():
    import torch  # noqa: F401
    from llama_decode_ubatch_amd import Model
    tens = {s.name: gen_tensor(WIDE, s) for s in tensor_specs(WIDE)}
    return tens, Model(WIDE, tens, device=0)


@pytest.mark.gpu
@pytest.mark.parametrize("n", [1, 2, 3])
def test_wide_rows_normalised_on_the_fly_when_the_stage_is_full(wide, n):
    tens, model = wide
    assert 4 * 1 * WIDE.n_embd <= 64 * 1024 < 4 * 2 * WIDE.n_embd
    run_both(model, WIDE, tens, rand_tokens(n, WIDE.n_vocab, seed=300 + n), 2, "f32", 1e-4, "wide")


@pytest.mark.gpu
@pytest.mark.parametrize("n", [1, 2])
def test_wide_rows_without_the_lds_stage(wide, n):
    """With the LDS-staged products switched off, the few-token kernel takes
    the norm: staged in LDS only for rows of at most 8192 values (what its
    prologue holds), normalised on the fly beyond that (9216 here)."""
    from llama_decode_ubatch_amd.binding import set_tuning
    tens, model = wide
    set_tuning("ldsx", 0)
    try:
        run_both(model, WIDE, tens, rand_tokens(n, WIDE.n_vocab, seed=320 + n), 2, "f32", 1e-4, "wide, ldsx off")
    finally:
        set_tuning("ldsx", 1)


def planted_tensors():
    tens = {s.name: gen_tensor(BIG, s) for s in tensor_specs(BIG)}
    for name in PLANTED:
        g = np.array(tens[name]["data"], np.float32)
        g[::32] = 1e5
        tens[name] = {"type": "f32", "data": g}
    return tens


@pytest.fixture(scope="module")
def big():
    import torch  # noqa: F401
    from llama_decode_ubatch_amd import Model
    tens = planted_tensors()
    return tens, Model(BIG, tens, device=0)


def test_planted_activations_pass_the_f16_range(monkeypatch):
    """CPU check of the fixture itself: in the oracle, the normalised inputs
    of the QKV product of layer 0 and of the logits product, and the SwiGLU
    output of layer 1 (the FFN down product's input), exceed 65504."""
    seen = {"norm": [], "swiglu": []}
    rms, swiglu = nm.rms_norm, nm.swiglu

    def rec_norm(*a, **k):
        y = rms(*a, **k)
        seen["norm"].append(float(np.abs(y).max()))
        return y

    def rec_swiglu(*a, **k):
        y = swiglu(*a, **k)
        seen["swiglu"].append(float(np.abs(y).max()))
        return y
    monkeypatch.setattr(nm, "rms_norm", rec_norm)
    monkeypatch.setattr(nm, "swiglu", rec_swiglu)
    tens = planted_tensors()
    ref = oracle_ctx(BIG, tens, np.float64, n_ctx=512, n_batch=512, n_ubatch=512, type_k="f32", type_v="f32")
    assert ref.decode(Batch(rand_tokens(4, BIG.n_vocab, seed=400), logits=[1] * 4)) == 0
    # norms in call order: layer 0 attention, layer 0 FFN, layer 1 attention,
    # layer 1 FFN, output
    assert len(seen["norm"]) == 5 and len(seen["swiglu"]) == 2
    assert seen["norm"][0] > F16_MAX and seen["norm"][3] > F16_MAX and seen["norm"][4] > F16_MAX
    assert seen["swiglu"][1] > F16_MAX


@pytest.mark.gpu
@pytest.mark.parametrize("n", [1, 2, 5])
def test_q8_0_products_rescale_rows_beyond_f16(big, n):
    tens, model = big
    run_both(model, BIG, tens, rand_tokens(n, BIG.n_vocab, seed=500 + n), 2, "f32", 2e-3, "q8_0 planted")
