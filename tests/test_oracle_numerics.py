"""Pins for oracle/numerics.py: closed forms, textbook special cases,
library routines and brute force (CPU only)."""
import math

import numpy as np
import pytest
from scipy.special import expit

from oracle import numerics as nm


def test_rmsnorm_constant_vector_closed_form():
    # RMSNorm of c*1 is c / sqrt(c^2 + eps) * g for every channel
    d, eps = 16, 1e-5
    g = np.linspace(0.5, 1.5, d)
    for c in (-3.0, 1e-3, 2.5):
        y = nm.rms_norm(np.full(d, c), g, eps)
        np.testing.assert_allclose(y, c / math.sqrt(c * c + eps) * g, rtol=1e-14)


def test_rmsnorm_output_mean_square():
    # with unit gain, mean(y^2) = m / (m + eps) where m = mean(x^2)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 33))
    y = nm.rms_norm(x, np.ones(33), 1e-3)
    m = np.mean(x * x, axis=1)
    np.testing.assert_allclose(np.mean(y * y, axis=1), m / (m + 1e-3), rtol=1e-13)


def test_rmsnorm_scale_invariance_and_gain_per_channel():
    rng = np.random.default_rng(1)
    x = rng.standard_normal(40)
    g = rng.standard_normal(40)
    a = nm.rms_norm(x, g, 0.0)
    np.testing.assert_allclose(nm.rms_norm(7.0 * x, g, 0.0), a, rtol=1e-13)
    # channel j of the output only depends on g[j]
    g2 = g.copy(); g2[3] *= 2
    b = nm.rms_norm(x, g2, 0.0)
    assert b[3] == pytest.approx(2 * a[3]) and np.array_equal(np.delete(a, 3), np.delete(b, 3))


def _rope_complex(x, pos, base):
    """Textbook RoPE: pair (2i, 2i+1) as the complex number x_2i + j x_2i+1
    multiplied by exp(j * pos * base^(-2i/hd))."""
    T, nh, hd = x.shape
    z = x[..., 0::2] + 1j * x[..., 1::2]
    theta = base ** (-np.arange(hd // 2) * 2.0 / hd)
    rot = np.exp(1j * pos[:, None, None] * theta[None, None, :])
    w = z * rot
    out = np.empty_like(x)
    out[..., 0::2] = w.real
    out[..., 1::2] = w.imag
    return out


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((6, 3, 8))
    pos = np.array([0, 1, 2, 17, 300, 4095])
    np.testing.assert_allclose(nm.rope_normal(x, pos, 10000.0),
                               _rope_complex(x, pos, 10000.0), atol=1e-12)


def test_rope_hand_values():
    # hd = 4: pair 0 turns by p, pair 1 by p * base^(-1/2)
    base = 10000.0
    x = np.array([[[1.0, 0.0, 1.0, 0.0]]])
    y = nm.rope_normal(x, np.array([3]), base)[0, 0]
    np.testing.assert_allclose(y, [math.cos(3), math.sin(3),
                                   math.cos(3 / 100.0), math.sin(3 / 100.0)], atol=1e-15)


def test_rope_identity_at_zero_and_norm_preserved():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 2, 32))
    np.testing.assert_array_equal(nm.rope_normal(x, np.zeros(4, int), 5e5), x)
    y = nm.rope_normal(x, np.array([5, 50, 500, 5000]), 5e5)
    np.testing.assert_allclose(np.linalg.norm(y[..., 0::2] + 1j * y[..., 1::2], axis=-1),
                               np.linalg.norm(x[..., 0::2] + 1j * x[..., 1::2], axis=-1), rtol=1e-13)


def test_rope_relative_position():
    # q.k after RoPE depends only on the position difference
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 1, 32)); k = rng.standard_normal((1, 1, 32))
    for base in (1e4, 5e5):
        ref = np.sum(nm.rope_normal(q, np.array([9]), base) * nm.rope_normal(k, np.array([4]), base))
        for delta in (1, 100, 30000):
            v = np.sum(nm.rope_normal(q, np.array([9 + delta]), base)
                       * nm.rope_normal(k, np.array([4 + delta]), base))
            assert v == pytest.approx(ref, rel=1e-9, abs=1e-12)


def test_silu_swiglu_against_library_sigmoid():
    x = np.linspace(-20, 20, 401)
    np.testing.assert_allclose(nm.silu(x), x * expit(x), rtol=1e-13, atol=1e-300)
    u = np.cos(x)
    np.testing.assert_allclose(nm.swiglu(x, u), x * expit(x) * u, rtol=1e-13, atol=1e-300)
    assert nm.silu(np.array([0.0]))[0] == 0.0
    h = 1e-6
    assert (nm.silu(np.array([h]))[0] - nm.silu(np.array([-h]))[0]) / (2 * h) == pytest.approx(0.5)


def _attention_bruteforce(q, K, V, visible, scale):
    nq, hd = q.shape
    out = np.zeros((nq, hd))
    for h in range(nq):
        s = [sum(q[h, d] * K[c, d] for d in range(hd)) * scale if visible[c] else None
             for c in range(K.shape[0])]
        m = max(v for v in s if v is not None)
        e = [math.exp(v - m) if v is not None else 0.0 for v in s]
        z = sum(e)
        for c in range(K.shape[0]):
            for d in range(hd):
                out[h, d] += e[c] / z * V[c, d]
    return out


def test_attention_bruteforce_and_row_sums():
    rng = np.random.default_rng(5)
    for n_cells in (1, 3, 11):
        q = rng.standard_normal((4, 8)); K = rng.standard_normal((n_cells, 8))
        V = rng.standard_normal((n_cells, 8))
        vis = rng.random(n_cells) < 0.7
        vis[rng.integers(n_cells)] = True
        out, p = nm.attention_heads(q, K, V, vis, 1 / math.sqrt(8))
        np.testing.assert_allclose(out, _attention_bruteforce(q, K, V, vis, 1 / math.sqrt(8)), atol=1e-13)
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)
        assert np.all(p[:, ~vis] == 0.0)


def test_attention_single_visible_cell_returns_v():
    rng = np.random.default_rng(6)
    q = rng.standard_normal((3, 16)); K = rng.standard_normal((5, 16)); V = rng.standard_normal((5, 16))
    vis = np.zeros(5, bool); vis[2] = True
    out, p = nm.attention_heads(q, K, V, vis, 0.25)
    np.testing.assert_array_equal(out, np.tile(V[2], (3, 1)))


def test_q8_0_dequant_hand_blocks():
    q = np.zeros((2, 64), np.int8)
    q[0, :32] = np.arange(-16, 16)
    q[0, 32:] = 127
    q[1, :32] = -127
    q[1, 32:] = np.arange(32) - 5
    sc = np.array([[0.5, 2 ** -12], [1.5, -0.25]], np.float16).view(np.uint16)
    w = nm.q8_0_dequant(q, sc)
    np.testing.assert_array_equal(w[0, :32], np.arange(-16, 16) * 0.5)
    np.testing.assert_array_equal(w[0, 32:], 127 * 2.0 ** -12)
    np.testing.assert_array_equal(w[1, :32], -127 * 1.5)
    np.testing.assert_array_equal(w[1, 32:], (np.arange(32) - 5) * -0.25)


def test_kv_rounding_is_ieee_half():
    x = np.array([1.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, 65504.0, 1e-8, -2.5])
    r = nm.round_to_kv_type(x, "f16").astype(np.float64)
    # ties to even: 1 + 2^-11 -> 1, 1 + 3*2^-11 -> 1 + 2^-9; subnormal flush of 1e-8 -> 0
    np.testing.assert_array_equal(r, [1.0, 1.0, 1.0 + 2 ** -9, 65504.0, 0.0, -2.5])
    assert nm.round_to_kv_type(x, "f32").dtype == np.float32


def test_bf16_upcast_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F7F], np.uint16)
    np.testing.assert_array_equal(nm.bf16_bits_to_f32(bits),
                                  np.array([1.0, -1.0, 3.140625, 0.0, 3.3895313892515355e38], np.float32))


# ------------------------------------------------------------ q8_0 KV blocks
def test_q8_0_quantize_exact_scale_block():
    # amax 127 gives d = 1 and 1/d = 1 exactly: codes are x rounded to
    # nearest with halves away from zero
    x = np.zeros(32, np.float32)
    x[:8] = [127.0, -127.0, 2.5, -2.5, 0.49, -0.51, 63.5, -0.5]
    codes, sc = nm.q8_0_quantize(x[None, :])
    assert codes[0, :8].tolist() == [127, -127, 3, -3, 0, -1, 64, -1]
    assert np.all(codes[0, 8:] == 0)
    assert nm.f16_bits_to_f32(sc)[0, 0] == 1.0


def test_q8_0_quantize_error_bound_and_range():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((64, 128)) * rng.uniform(1e-3, 10, (64, 1))).astype(np.float32)
    codes, sc = nm.q8_0_quantize(x)
    assert codes.min() >= -127 and codes.max() <= 127
    # every block reaches +-127 at its largest magnitude
    assert np.all(np.abs(codes.reshape(64, 4, 32)).max(-1) == 127)
    d = np.abs(x.reshape(64, 4, 32)).max(-1) / 127
    y = nm.q8_0_dequant(codes, sc)
    # rounding to the code grid (half a step) plus the f16 rounding of the scale
    err = np.abs(y - x).reshape(64, 4, 32).max(-1)
    assert np.all(err <= d * (0.5 + 127 * 2.0 ** -11) * (1 + 1e-6))
    # stored value = round_to_kv_type
    assert np.array_equal(nm.round_to_kv_type(x, "q8_0"), y)


def test_q8_0_quantize_zero_block():
    codes, sc = nm.q8_0_quantize(np.zeros((2, 64), np.float32))
    assert not codes.any() and not sc.any()
    assert not nm.round_to_kv_type(np.zeros((2, 64), np.float32), "q8_0").any()


def test_q8_0_quantize_rejects_planted_offset():
    # a quantiser that forgot the sign of the halves would fail the tie case
    x = np.zeros(32, np.float32)
    x[0], x[1] = 127.0, -2.5
    codes, _ = nm.q8_0_quantize(x[None, :])
    assert codes[0, 1] == -3 and np.trunc(-2.5 + 0.5) != -3
