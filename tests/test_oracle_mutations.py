"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and
check that the independent pins catch every one of them."""
import math

import numpy as np
import pytest

from oracle import numerics as nm
from tests import test_oracle_model as tm
from tests.helpers import MICRO, oracle_ctx, rand_tokens


def _neox_rope(x, pos, base):
    # pairs (i, i + hd/2) instead of (2i, 2i+1)
    T, nh, hd = x.shape
    h = hd // 2
    inv = base ** (-2.0 * np.arange(h) / hd)
    a = pos[:, None, None] * inv
    x0, x1 = x[..., :h], x[..., h:]
    return np.concatenate([x0 * np.cos(a) - x1 * np.sin(a), x0 * np.sin(a) + x1 * np.cos(a)], -1)


def _rope_wrong_sign(x, pos, base):
    return ORIG_ROPE(x, -pos, base)


def _attention_no_scale(q, K, V, visible, scale):
    return ORIG_ATT(q, K, V, visible, 1.0)


def _attention_no_mask(q, K, V, visible, scale):
    return ORIG_ATT(q, K, V, np.ones_like(visible), scale)


def _swapped_swiglu(gate, up):
    return ORIG_SWIGLU(up, gate)


def _rms_eps_outside(x, g, eps):
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * g


def _rms_no_gain(x, g, eps):
    return ORIG_RMS(x, np.ones_like(g), eps)


ORIG_ATT = nm.attention_heads
ORIG_SWIGLU = nm.swiglu
ORIG_RMS = nm.rms_norm
ORIG_ROPE = nm.rope_normal

MUTANTS = {
    "rope_neox_pairing": ("rope_normal", _neox_rope),
    "rope_wrong_sign": ("rope_normal", _rope_wrong_sign),
    "attention_no_scale": ("attention_heads", _attention_no_scale),
    "attention_no_mask": ("attention_heads", _attention_no_mask),
    "swiglu_swapped": ("swiglu", _swapped_swiglu),
    "rms_no_gain": ("rms_norm", _rms_no_gain),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_brute_force_catches_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(nm, attr, fn)
    toks = rand_tokens(9, MICRO.n_vocab, 2)
    a = tm._prefill_all(oracle_ctx(tensors=tm.TENS, n_ubatch=4), toks)
    ref = tm._brute_forward(MICRO, tm.TENS, toks)
    assert np.abs(a - ref).max() > 1e-6 * np.abs(ref).max()


def test_eps_placement_caught_by_closed_form(monkeypatch):
    monkeypatch.setattr(nm, "rms_norm", _rms_eps_outside)
    from tests import test_oracle_numerics as tn
    with pytest.raises(AssertionError):
        tn.test_rmsnorm_constant_vector_closed_form()
