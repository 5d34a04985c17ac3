"""On-device sampler chain against the oracle's (engine page, Steps 14-16,
"Sampler chain").

Both sides get the same float32 logits.  The GPU computes in float32 and the
oracle in float64, so a draw is compared only where u lies further than
1e-5 from a boundary of the accumulated probabilities (the margin the oracle
reports); the candidate list (ids, in order) must match exactly and the
probabilities within 1e-5.  Rows: seeded normal logits, rows with planted
exact ties (at the top and at the top-k boundary), an all-equal row (more
ties than the kernel's candidate list holds), vocabularies from 1 token to
152k, and the logits rows of a tiny model's decode.
"""
import numpy as np
import pytest

from oracle.sampling import SamplerParams, candidates, sample

pytestmark = pytest.mark.gpu

PARAMS = {
    "default": dict(),
    "greedy-k1": dict(top_k=1),
    "temp0": dict(top_k=100, temperature=0.0),
    "top_p": dict(top_k=200, top_p=0.9),
    "min_p": dict(top_k=200, min_p=0.05),
    "hot": dict(top_k=1024, temperature=1.7),
    "cold-mixed": dict(top_k=64, top_p=0.95, min_p=0.02, temperature=0.6),
    "penalties": dict(top_k=50, penalty_last_n=64, penalty_repeat=1.3, penalty_freq=0.2, penalty_present=0.1),
    "penalty-raises": dict(top_k=50, penalty_last_n=256, penalty_repeat=0.7, penalty_freq=-0.3),
}


@pytest.fixture(scope="module")
def env():
    import torch
    from llama_decode_ubatch_amd import Model, Context
    from workloads import MODELS, gen_tensor, tensor_specs
    shape = MODELS["tiny-f32"]
    tens = {s.name: gen_tensor(shape, s) for s in tensor_specs(shape)}
    model = Model(shape, tens, device=0)
    ctx = Context(model, n_ctx=512, n_batch=512, n_ubatch=64, n_seq_max=4)
    return torch, shape, tens, model, ctx


def check_draw(smpl, run, z, hist, p, u, label):
    """run(u) draws on the GPU; compare it with the oracle on logits z."""
    t = run(u)
    tr, margin = sample(z, hist, p, u)
    c, v = candidates(z, hist, p)
    ids, probs = smpl.candidates()
    np.testing.assert_array_equal(ids, c.astype(np.int32), err_msg=label)
    if p.temperature > 0:
        pr = np.exp(v - v.max())
        pr /= pr.sum()
    else:
        pr = (np.arange(c.size) == 0).astype(np.float64)
    np.testing.assert_allclose(probs, pr, atol=1e-5, rtol=0, err_msg=label)
    if margin > 1e-5:
        assert t == tr, f"{label}: u={u} gpu {t} oracle {tr} (margin {margin:.2e})"
    else:
        assert t in c, label
    return t


def rows(rng, V):
    z = (rng.standard_normal(V) * 3).astype(np.float32)
    yield "normal", z
    if V >= 60:
        zt = z.copy()
        top = np.argsort(-zt, kind="stable")
        zt[top[:5]] = zt[top[0]]                # five-way tie at the top
        zt[top[45:60]] = zt[top[50]]            # ties across the top-k boundary
        yield "ties", zt
    yield "heavy", (rng.standard_t(2, V) * 2).astype(np.float32)


@pytest.mark.parametrize("V", [1, 7, 1000, 128256])
@pytest.mark.parametrize("name", list(PARAMS))
def test_sampler_matches_oracle(env, V, name):
    torch, _, _, _, ctx = env
    from llama_decode_ubatch_amd import Sampler
    p = SamplerParams(**PARAMS[name])
    rng = np.random.default_rng(V * 31 + len(name))
    for kind, z in rows(rng, V):
        dz = torch.from_numpy(z).to("cuda:0")
        torch.cuda.synchronize()
        hist = rng.integers(0, V, 300).tolist() if p.penalty_last_n else []
        for u in (0.0, 0.37, 0.9999, *rng.random(3).tolist()):
            smpl = Sampler(ctx, **PARAMS[name])
            smpl.accept(hist)
            check_draw(smpl, lambda u: smpl.sample_logits(dz, u), z, hist, p, u, f"{name} V={V} {kind} u={u}")
            smpl.free()


def test_sampler_history_grows_with_its_draws(env):
    """Each draw joins the history, so penalties act on the sampler's own
    earlier choices."""
    torch, _, _, _, ctx = env
    from llama_decode_ubatch_amd import Sampler
    prm = dict(top_k=20, temperature=0.8, penalty_last_n=8, penalty_repeat=1.5, penalty_present=0.5)
    p = SamplerParams(**prm)
    rng = np.random.default_rng(9)
    z = (rng.standard_normal(5000) * 2).astype(np.float32)
    dz = torch.from_numpy(z).to("cuda:0")
    torch.cuda.synchronize()
    smpl = Sampler(ctx, **prm)
    hist = [3, 3, 17]
    smpl.accept(hist)
    for step in range(40):
        t = check_draw(smpl, lambda u: smpl.sample_logits(dz, u), z, hist, p, float(rng.random()), f"step {step}")
        hist.append(t)
    smpl.free()


def test_all_equal_row_overflows_the_candidate_list(env):
    torch, _, _, _, ctx = env
    from llama_decode_ubatch_amd import Sampler
    z = np.zeros(20000, np.float32)
    dz = torch.from_numpy(z).to("cuda:0")
    torch.cuda.synchronize()
    for prm in (dict(top_k=40), dict(top_k=1024, top_p=0.5), dict(top_k=5, penalty_last_n=4, penalty_repeat=0.5,
                                                                    penalty_present=-1.0)):
        p = SamplerParams(**prm)
        smpl = Sampler(ctx, **prm)
        hist = [19999, 12, 12, 4000]
        smpl.accept(hist)
        check_draw(smpl, lambda u: smpl.sample_logits(dz, u), z, hist, p, 0.5, str(prm))
        smpl.free()


def test_sampler_on_decode_rows(env):
    """Rows of the context's own logits (ubd_sampler_sample with a batch
    index), four sequences in one decode."""
    _, shape, _, _, ctx = env
    from llama_decode_ubatch_amd import Sampler
    rng = np.random.default_rng(4)
    toks = rng.integers(0, shape.n_vocab, 4 * 20).astype(np.int32)
    seqs = np.repeat(np.arange(4), 20).astype(np.int32)
    flags = np.zeros(toks.size, np.int8)
    flags[19::20] = 1
    ctx.seq_rm(-1, -1, -1)
    assert ctx.decode(toks, seq_id=seqs, logits=flags) == 0
    prm = dict(top_k=40, top_p=0.95, temperature=0.9)
    p = SamplerParams(**prm)
    smpl = Sampler(ctx, **prm)
    for b in np.nonzero(flags)[0]:
        z = ctx.logits_ith(int(b))
        for u in rng.random(4):
            check_draw(smpl, lambda u: smpl.sample(int(b), float(u)), z, [], p, float(u), f"row {b}")
    assert smpl.sample(3, 0.5) == -1            # not an output row
    assert smpl.sample(int(b), 1.0) == -1       # u out of range
    smpl.free()


def test_sampler_rejects_bad_parameters(env):
    _, _, _, _, ctx = env
    from llama_decode_ubatch_amd import Sampler
    for bad in (dict(top_k=0), dict(top_k=1025), dict(top_p=0.0), dict(top_p=1.5), dict(min_p=1.0),
                dict(penalty_last_n=257), dict(penalty_repeat=0.0)):
        with pytest.raises(ValueError):
            Sampler(ctx, **bad)
