"""Prefill products at small, ragged shapes, through the C ABI.

Small Llama-architecture models with bf16 and q8_0 weights (the tiny
workloads use f32 weights, which never take the MFMA GEMM path) prefill
prompts of 64, 100 and 200 tokens with every token flagged for output, so
the QKV, O, gate|up, down and logits products all run as GEMMs with a
ragged token tail, weight-row tiles that overhang N, k both a multiple of 128
and not (n_ff 704), and split-k residual products (n_ff 1408; n_ff 1536 for
the split through scratch).  All logits
are compared with the float64 oracle; the LDS-ring kernel is also compared
with the register-staged one.  Ubatches of 1, 2, 5 and 16 tokens run the
same models through the decode products instead.
"""
import numpy as np
import pytest

from workloads import ModelShape, gen_tensor, tensor_specs
from tests.helpers import oracle_ctx, rand_tokens

pytestmark = pytest.mark.gpu

SHAPES = {
    "bf16-ff1408": ModelShape("small-bf16-a", 10, n_layer=2, n_embd=256, n_head=8, n_head_kv=2, n_ff=1408,
                              n_vocab=1024, n_ctx_train=2048, rope_base=10000.0, wtype="bf16"),
    "bf16-ff704": ModelShape("small-bf16-b", 11, n_layer=2, n_embd=256, n_head=8, n_head_kv=2, n_ff=704,
                             n_vocab=1024, n_ctx_train=2048, rope_base=10000.0, wtype="bf16"),
    # k = 1536 splits into two slices of 12 stages: the forced deep shapes
    # then run the residual products split over k through scratch
    "bf16-ff1536": ModelShape("small-bf16-c", 13, n_layer=2, n_embd=256, n_head=8, n_head_kv=2, n_ff=1536,
                              n_vocab=1024, n_ctx_train=2048, rope_base=10000.0, wtype="bf16"),
    "q8_0-ff1408": ModelShape("small-q8-a", 12, n_layer=2, n_embd=256, n_head=8, n_head_kv=2, n_ff=1408,
                              n_vocab=1024, n_ctx_train=2048, rope_base=10000.0, wtype="q8_0"),
}
# the products see the activations as hi + lo planes (about 16 significant
# bits); with the bf16 prefill products on the hi plane alone (bf16-rounded
# activations) the bf16 tolerance is 3e-2
TOL = {"bf16": 2e-3, "q8_0": 2e-3}
TOL_HI_ONLY = 3e-2


@pytest.fixture(scope="module")
def built():
    import torch  # noqa: F401
    from llama_decode_ubatch_amd import Model
    out = {}
    for key, shape in SHAPES.items():
        tens = {s.name: gen_tensor(shape, s) for s in tensor_specs(shape)}
        out[key] = (shape, tens, Model(shape, tens, device=0))
    return out


def gpu_logits(model, tokens, gemm, shape=0, tiled=1, lo=1, split=0):
    from llama_decode_ubatch_amd import Context
    from llama_decode_ubatch_amd.binding import set_tuning
    set_tuning("gemm", gemm)
    set_tuning("gemm_shape", shape)
    set_tuning("act_tiled", tiled)
    set_tuning("prefill_lo", 31 if lo else 0)
    set_tuning("gemm_split", split)
    try:
        ctx = Context(model, n_ctx=512, n_batch=512, n_ubatch=512, n_seq_max=1, type_k="f16", type_v="f16")
        assert ctx.decode(tokens, logits=np.ones(len(tokens))) == 0
        return ctx.logits()
    finally:
        set_tuning("gemm", 1)
        set_tuning("gemm_shape", 0)
        set_tuning("act_tiled", 1)
        set_tuning("prefill_lo", 31)
        set_tuning("gemm_split", 0)


@pytest.mark.parametrize("key", list(SHAPES))
@pytest.mark.parametrize("n", [64, 100, 200])
def test_prefill_gemm_matches_oracle(built, key, n):
    shape, tens, model = built[key]
    tokens = rand_tokens(n, shape.n_vocab, seed=1000 + n)
    z = gpu_logits(model, tokens, 1)
    ref = oracle_ctx(shape, tens, np.float64, n_ctx=512, n_batch=512, n_ubatch=512, type_k="f16", type_v="f16")
    from oracle import Batch
    assert ref.decode(Batch(tokens, logits=[1] * n)) == 0
    zr = np.stack([ref.logits_ith(i) for i in range(n)])
    err = float(np.abs(z - zr).max() / np.abs(zr).max())
    print(f"{key} T={n}: logits rel err {err:.2e}", flush=True)
    assert err < TOL[shape.wtype]
    # the other kernel choices must sit within the tolerance too: with both
    # activation planes, each forced tile of the LDS-ring and deep kernels
    # (bf16: 1, 3, 5, 10, 14, 16, 18 to 25; q8_0: every LDS-ring tile) and row-major
    # activations; with the hi plane alone (bf16), the register-staged kernel
    # and every tile of the two kernels
    lo_choices = [(1, c) for c in (1, 2, 3, 4, 5, 10, 14, 16, 18, 19, 20, 21, 22, 23, 24, 25)] + [(1, 0, 0), (1, 10, 0)]
    for choice in lo_choices:
        zc = gpu_logits(model, tokens, *choice)
        assert float(np.abs(zc - zr).max() / np.abs(zr).max()) < TOL[shape.wtype], choice
    # residual products split over k into 2 and 4 slices (added in slice
    # order, so two runs give the same logits bit for bit)
    for split in (2, 4):
        zc = gpu_logits(model, tokens, 1, split=split, lo=0 if shape.wtype == "bf16" else 1)
        tol = TOL_HI_ONLY if shape.wtype == "bf16" else TOL[shape.wtype]
        assert float(np.abs(zc - zr).max() / np.abs(zr).max()) < tol, split
        assert np.array_equal(zc, gpu_logits(model, tokens, 1, split=split, lo=0 if shape.wtype == "bf16" else 1))
    if shape.wtype == "bf16":
        for choice in ((0, 0), (1, 0), (1, 1), (1, 2), (1, 3), (1, 4), (1, 7), (1, 8), (1, 9), (1, 10), (1, 11), (1, 12),
                       (1, 13), (1, 14), (1, 15), (1, 0, 0), (1, 10, 0)):
            zc = gpu_logits(model, tokens, *(choice + (1,) * (3 - len(choice))), lo=0)
            assert float(np.abs(zc - zr).max() / np.abs(zr).max()) < TOL_HI_ONLY, choice


@pytest.mark.parametrize("key", list(SHAPES))
@pytest.mark.parametrize("n", [1, 2, 5, 16])
def test_few_token_products_match_oracle(built, key, n):
    """Fewer than 64 tokens take the decode products instead of the GEMMs:
    the LDS-staged kernel where a 16-token block's activations fit its stage
    (k = 256 here; the RMSNorm fused into it for at most 2 tokens) and the
    kernel that reads the activations from L2 otherwise (the down product,
    k = n_ff).  Every logits row is compared with the float64 oracle."""
    shape, tens, model = built[key]
    tokens = rand_tokens(n, shape.n_vocab, seed=2000 + n)
    z = gpu_logits(model, tokens, 1)
    ref = oracle_ctx(shape, tens, np.float64, n_ctx=512, n_batch=512, n_ubatch=512, type_k="f16", type_v="f16")
    from oracle import Batch
    assert ref.decode(Batch(tokens, logits=[1] * n)) == 0
    zr = np.stack([ref.logits_ith(i) for i in range(n)])
    err = float(np.abs(z - zr).max() / np.abs(zr).max())
    print(f"{key} T={n}: logits rel err {err:.2e}", flush=True)
    assert err < TOL[shape.wtype]


def prefill_with_norm_counts(model, tokens, split, lo, post_norm):
    """Logits of a 100-token prefill and the prefill RMSNorm launches that ran
    as kernels of their own."""
    from llama_decode_ubatch_amd import Context
    from llama_decode_ubatch_amd.binding import set_tuning
    set_tuning("gemm_split", split)
    set_tuning("prefill_lo", 31 if lo else 0)
    set_tuning("post_norm", post_norm)
    try:
        ctx = Context(model, n_ctx=512, n_batch=512, n_ubatch=512, n_seq_max=1, type_k="f16", type_v="f16")
        ctx.kernel_timing(None)
        ctx.kernel_stats()
        assert ctx.decode(tokens, logits=np.ones(len(tokens))) == 0
        stats = ctx.kernel_stats()
        return ctx.logits(), stats.get("prefill.rmsnorm", (0, 0.0))[0]
    finally:
        set_tuning("gemm_split", 0)
        set_tuning("prefill_lo", 31)
        set_tuning("post_norm", 1)


@pytest.mark.parametrize("key", list(SHAPES))
def test_norm_in_the_k_slice_pass_is_bit_identical(built, key):
    """A residual product whose k is split adds its slices into the residual
    in a pass that also runs the RMSNorm after it (the FFN norm after O, the
    next layer's attention norm after down).  With the products forced into
    2 and 4 slices, that pass replaces those norm kernels (one attention norm
    of the first layer and the output norm remain) and the logits equal those
    with every norm in its own kernel, bit for bit."""
    shape, tens, model = built[key]
    tokens = rand_tokens(100, shape.n_vocab, seed=77)
    # (forced splits reach both residual products on the bf16 hi-plane path
    # and the q8_0 path at these shapes)
    lo = 0 if shape.wtype == "bf16" else 1
    cases = [(2, lo), (4, lo)]
    for split, lo in cases:
        print(f"{key}: k in {split} slices, lo plane {lo}", flush=True)
        fused, n_fused = prefill_with_norm_counts(model, tokens, split, lo, 1)
        sep, n_sep = prefill_with_norm_counts(model, tokens, split, lo, 0)
        assert n_sep == 2 * shape.n_layer + 1
        assert n_fused == 2, n_fused
        assert np.array_equal(fused, sep), (split, lo)
