"""Pins for the oracle's logit decoding and target softmax.

Fixed by mathematics and by library routines independent of the oracle:
bf16 bit patterns with known values, scipy's softmax and logsumexp, the
two-token logistic closed form, shift invariance and the T -> scaling rule.
"""
import numpy as np
import pytest
from scipy.special import logsumexp, softmax

from oracle import decode_logits, first_argmax, target_distribution


def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x7F80, 0xFF80, 0x0001, 0x8000, 0x4049, 0x0000],
                    dtype=np.uint16)
    want = [1.0, -2.0, np.inf, -np.inf, 2.0 ** -133, -0.0, 3.140625, 0.0]
    got = decode_logits(bits, "bf16")
    assert got.dtype == np.float64
    for g, w in zip(got, want):
        assert g == w and np.signbit(g) == np.signbit(w)


def test_f32_decode_is_exact_widening():
    x = np.array([1e-45, 3.4028235e38, -0.1, 7.0], dtype=np.float32)
    assert np.array_equal(decode_logits(x, "f32"), x.astype(np.float64))


@pytest.mark.parametrize("T", [1.0, 0.7, 0.25, 3.0])
@pytest.mark.parametrize("V", [1, 2, 7, 1000, 32000])
def test_softmax_matches_scipy(T, V):
    rng = np.random.default_rng(V * 17 + int(T * 100))
    z = 3.0 * rng.standard_normal(V)
    p = target_distribution(z, T)
    assert np.allclose(p, softmax(z / T), rtol=1e-13, atol=0.0)
    assert abs(p.sum() - 1.0) < 1e-13
    # log p = z/T - logsumexp(z/T)
    nz = p > 0
    assert np.allclose(np.log(p[nz]), (z / T - logsumexp(z / T))[nz], rtol=0, atol=1e-11)


def test_two_token_logistic():
    for z0, z1, T in [(0.0, 1.0, 1.0), (3.5, -2.0, 0.7), (10.0, 10.0, 2.0)]:
        p = target_distribution(np.array([z0, z1]), T)
        want0 = 1.0 / (1.0 + np.exp((z1 - z0) / T))
        assert abs(p[0] - want0) < 1e-15 and abs(p[1] - (1 - want0)) < 1e-15


def test_shift_invariance_and_neg_inf():
    rng = np.random.default_rng(3)
    z = rng.standard_normal(50)
    z[[3, 9]] = -np.inf
    p = target_distribution(z, 0.9)
    assert p[3] == 0.0 and p[9] == 0.0
    assert np.allclose(p, target_distribution(z + 123.25, 0.9), rtol=1e-12, atol=0)
    # large logits do not overflow
    assert np.allclose(target_distribution(z + 1e4, 0.9), p, rtol=1e-9, atol=0)


def test_temperature_is_power_rule():
    # softmax(z/T) is proportional to softmax(z)^(1/T)
    rng = np.random.default_rng(4)
    z = rng.standard_normal(40)
    p1 = target_distribution(z, 1.0)
    pT = target_distribution(z, 0.5)
    w = p1 ** 2.0
    assert np.allclose(pT, w / w.sum(), rtol=1e-12, atol=0)


def test_first_argmax_ties_and_library():
    z = np.array([1.0, 5.0, -2.0, 5.0, 5.0])
    assert first_argmax(z) == 1
    z2 = np.array([-0.0, 0.0, -1.0])          # -0 == +0: the first one wins
    assert first_argmax(z2) == 0
    z3 = np.full(6, -np.inf)
    assert first_argmax(z3) == 0
    rng = np.random.default_rng(5)
    for _ in range(200):
        x = rng.integers(-3, 3, size=rng.integers(1, 20)).astype(np.float64)
        # brute force: smallest index among those equal to the max
        assert first_argmax(x) == min(i for i, v in enumerate(x) if v == x.max())
