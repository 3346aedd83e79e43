"""Exact pins for the oracle's sampled verify.

The law of the oracle's outputs is measured by bisection over the uniforms
(the oracle used as a black box) and compared with the closed-form law of
speculative sampling (see tests/pins.py).  A dropped max(0, .), a wrong row
index, a wrong sign or a swapped p/q changes that law.  Special cases reduce to
known answers; the inverse-CDF draw is compared with numpy.searchsorted.
"""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import verify_sample, verify_sample_seq
from oracle.verify import accept_ratio, inverse_cdf
from tests.pins import blackbox_law, closed_form_law, law_distance, random_case


def oracle_ac(z, q, d, u, T):
    tr = verify_sample_seq(z, q, d, u, T)
    return tr.a, tr.c


@pytest.mark.parametrize("V,K,T,seed,zero_q,neg_inf", [
    (3, 1, 1.0, 0, False, False),
    (4, 2, 1.0, 1, False, False),
    (4, 2, 0.7, 2, True, False),
    (5, 1, 1.7, 3, False, True),
    (3, 3, 1.0, 4, True, True),
])
def test_exact_law(V, K, T, seed, zero_q, neg_inf):
    rng = np.random.default_rng(seed)
    z, q = random_case(rng, V, K, zero_q=zero_q, neg_inf=neg_inf)
    got = blackbox_law(oracle_ac, z, q, T)
    want = closed_form_law(z, q, T)
    assert abs(sum(got.values()) - 1.0) < 1e-12
    assert law_distance(got, want) < 1e-12
    # lossless: the first emitted token is distributed as p_0
    first = np.zeros(V)
    for key, w in got.items():
        a = key[0]
        first[key[1] if a > 0 else key[1 + a]] += w
    assert np.allclose(first, softmax(z[0] / T), rtol=0, atol=1e-12)


def test_q_equals_p_accepts_everything():
    rng = np.random.default_rng(21)
    K, V = 3, 6
    z = rng.standard_normal((K + 1, V))
    q = np.stack([softmax(z[k]) for k in range(K)])           # exactly p (T = 1)
    for _ in range(200):
        u = rng.random(K + 1)
        tr = verify_sample_seq(z, q, [int(rng.integers(V)) for _ in range(K)], u, 1.0)
        assert tr.a == K
    # and the bonus follows p_K: its law is exactly softmax(z_K)
    law = blackbox_law(oracle_ac, z, q, 1.0)
    bonus = np.zeros(V)
    for key, w in law.items():
        assert key[0] == K
        bonus[key[-1]] += w
    assert np.allclose(bonus, softmax(z[K]), atol=1e-12)


def test_q_one_hot_on_zero_of_p_always_rejects():
    z = np.array([[0.0, -np.inf, 1.0, 0.5], [0.0, 0.0, 0.0, 0.0]])
    q = np.array([[0.0, 1.0, 0.0, 0.0]])                      # drafter is sure of token 1
    law = blackbox_law(oracle_ac, z, q, 1.0)
    p0 = softmax(z[0])
    for key, w in law.items():
        assert key[0] == 0
    got = np.zeros(4)
    for key, w in law.items():
        got[key[1]] += w
    assert np.allclose(got, p0, atol=1e-12)                   # residual = p_0


def test_disjoint_supports():
    z = np.array([[0.0, 0.0, -np.inf, -np.inf], [1.0, 2.0, 3.0, 4.0]])
    q = np.array([[0.0, 0.0, 0.5, 0.5]])
    for d in (2, 3):
        for u in (0.0, 0.3, 0.99):
            tr = verify_sample_seq(z, q, [d], [u, 0.4], 1.0)
            assert tr.a == 0 and tr.c in (0, 1)


def test_unnormalised_q_falls_back_to_p():
    # q = 2p: ratio 1/2 everywhere and the residual max(0, p - 2p) is zero
    z = np.array([[0.0, 1.0, 2.0], [0.0, 0.0, 0.0]])
    p = softmax(z[0])
    q = 2.0 * p[None, :]
    tr = verify_sample_seq(z, q, [2], [0.75, 0.5], 1.0)
    assert tr.a == 0 and tr.draw_from_p
    c, _, _ = inverse_cdf(p, 0.5)
    assert tr.c == c
    tr2 = verify_sample_seq(z, q, [2], [0.25, 0.5], 1.0)
    assert tr2.a == 1


def test_accept_ratio_zero_q():
    assert accept_ratio(0.3, 0.0) == np.inf
    assert accept_ratio(0.0, 0.0) == 0.0
    assert accept_ratio(0.2, 0.4) == 0.5


def test_inverse_cdf_matches_searchsorted():
    rng = np.random.default_rng(8)
    for _ in range(500):
        V = int(rng.integers(1, 40))
        r = rng.random(V) * (rng.random(V) < 0.6)
        if r.sum() == 0:
            r[rng.integers(V)] = 0.3
        u = float(rng.random())
        c, S, cdf = inverse_cdf(r, u)
        want = int(np.searchsorted(np.cumsum(r), u * np.cumsum(r)[-1], side="right"))
        assert c == want
        assert r[c] > 0.0
    # zero-mass tokens are never returned, also at the cell edges
    r = np.array([0.0, 0.5, 0.0, 0.5, 0.0])
    for u in [0.0, 0.5, np.nextafter(0.5, 0), np.nextafter(1.0, 0)]:
        c, _, _ = inverse_cdf(r, u)
        assert r[c] > 0


def test_batch_api_matches_sequences():
    rng = np.random.default_rng(9)
    B, K, V = 6, 4, 20
    z = (2.0 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    q = softmax(z[:, :K].astype(np.float64) + rng.standard_normal((B, K, V)), axis=2).astype(np.float32)
    d = np.array([[rng.choice(V, p=q[b, k] / q[b, k].sum()) for k in range(K)] for b in range(B)],
                 dtype=np.int32)
    u = rng.random((B, K + 1), dtype=np.float32)
    out, acc, pd = verify_sample(z, "f32", q, d, u, 0.8)
    for b in range(B):
        tr = verify_sample_seq(z[b].astype(np.float64), q[b], d[b], u[b], 0.8)
        assert acc[b] == tr.a and np.array_equal(out[b], tr.out_tokens)
        p = [softmax(z[b, k].astype(np.float64) / 0.8) for k in range(K)]
        assert np.allclose(pd[b], [p[k][d[b, k]] for k in range(K)], rtol=1e-13, atol=0)
        assert np.all(out[b, acc[b] + 1:] == -1)
        assert np.array_equal(out[b, :acc[b]], d[b, :acc[b]])
