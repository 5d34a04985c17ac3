"""Pins of the oracle's sampler chain (engine page, Steps 14-16, "Sampler
chain"): closed forms and special cases that reduce to greedy choice or to
an inverse-CDF draw, on hand-built distributions."""
import numpy as np
import pytest

from oracle.sampling import SamplerParams, apply_penalties, candidates, sample

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def logp(probs):
    return np.log(np.asarray(probs, np.float64))


def test_greedy_special_cases():
    rng = np.random.default_rng(3)
    z = rng.standard_normal(5000)
    z[4000] = z[17] = z.max() + 1.0            # tie at the top: lower id wins
    for p in (SamplerParams(top_k=1), SamplerParams(top_k=1000, temperature=0.0)):
        for u in (0.0, 0.5, 0.999):
            assert sample(z, [], p, u)[0] == 17


def test_inverse_cdf_with_no_cut():
    probs = np.array([0.1, 0.4, 0.2, 0.3])
    p = SamplerParams(top_k=4)
    order = [1, 3, 2, 0]                       # by probability descending
    cum = np.cumsum(probs[order])
    for i, t in enumerate(order):
        lo = cum[i - 1] if i else 0.0
        assert sample(logp(probs), [], p, (lo + cum[i]) / 2)[0] == t


def test_penalty_closed_forms():
    z = np.array([2.0, -2.0, 0.5, 1.0])
    p = SamplerParams(penalty_last_n=8, penalty_repeat=2.0, penalty_freq=0.25, penalty_present=0.5)
    out = apply_penalties(z, [0, 1, 1, 3, 3, 3], p)
    assert np.allclose(out, [2.0 / 2 - 0.25 - 0.5, -4.0 - 0.5 - 0.5, 0.5, 0.5 - 0.75 - 0.5])
    # only the last penalty_last_n tokens count
    p2 = SamplerParams(penalty_last_n=2, penalty_repeat=2.0)
    assert np.allclose(apply_penalties(z, [0, 3, 1], p2), [2.0, -4.0, 0.5, 0.5])


def test_top_p_and_min_p_cut_offs():
    z = logp([0.5, 0.3, 0.2])
    ids = lambda p: candidates(z, [], p)[0].tolist()
    assert ids(SamplerParams(top_k=3, top_p=0.6)) == [0, 1]       # 0.5 < 0.6 <= 0.8
    assert ids(SamplerParams(top_k=3, top_p=0.5)) == [0]          # the first reaches 0.5
    assert ids(SamplerParams(top_k=3, top_p=0.95)) == [0, 1, 2]
    assert ids(SamplerParams(top_k=3, min_p=0.5)) == [0, 1]       # keep p >= 0.25
    assert ids(SamplerParams(top_k=3, min_p=0.7)) == [0]


def test_top_k_comes_before_top_p():
    # after top-k 2 the probabilities renormalise to 0.625 / 0.375, so top-p
    # 0.6 keeps one token; on the full set it would keep two
    z = logp([0.5, 0.3, 0.2])
    assert candidates(z, [], SamplerParams(top_k=2, top_p=0.6))[0].tolist() == [0]
    assert candidates(z, [], SamplerParams(top_k=3, top_p=0.6))[0].tolist() == [0, 1]


def test_temperature_is_a_power_of_the_probabilities():
    probs = np.array([0.5, 0.3, 0.2])
    c, v = candidates(logp(probs), [], SamplerParams(top_k=3, temperature=2.0))
    q = np.exp(v - v.max())
    q /= q.sum()
    ref = np.sqrt(probs) / np.sqrt(probs).sum()
    assert np.allclose(q, ref[c])


def test_draws_are_valid_candidates():
    rng = np.random.default_rng(5)
    z = rng.standard_normal(3000) * 3
    p = SamplerParams(top_k=50, top_p=0.9, min_p=0.05, temperature=0.8, penalty_last_n=16, penalty_repeat=1.3)
    hist = rng.integers(0, 3000, 40).tolist()
    c, _ = candidates(z, hist, p)
    for u in rng.random(200):
        t, margin = sample(z, hist, p, u)
        assert t in c.tolist() and margin >= 0
