"""Exact pins for the oracle's sampled verify.

The law of the oracle's outputs is measured by bisection over the uniforms
(the oracle used as a black box) and compared with the closed-form law of
speculative sampling (see tests/pins.py).  A dropped max(0, .), a wrong row
index, a wrong sign or a swapped p/q changes that law.  Special cases reduce to
known answers; the inverse-CDF draw is compared with numpy.searchsorted.
"""
import itertools

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


# ---------------------------------------------------------------- near-tie enumerator
# oracle.sample_outcomes lists the outcomes a correct evaluation may reach
# when a decision lies within tol of its threshold: an accept test with
# |u_k - p_k(x)/q_k(x)| < tol may go either way, and a final draw whose u*S
# lies within tol of a CDF boundary may return either neighbour with positive
# mass.  Every sampled GPU parity check accepts a result only if it is in
# that list, so the list is pinned here against quantities computed outside
# the oracle: p from scipy's softmax, the decision paths from the oracle's
# forced-decision replay (verify_sample_seq(force=...)), and the draw band by
# brute force over perturbed uniforms.

def _p_rows(z, T):
    return [softmax(np.asarray(z[k], np.float64) / T) for k in range(z.shape[0])]


def _ratio(p, q, x):
    if q[x] > 0.0:
        return p[x] / q[x]
    return np.inf if p[x] > 0.0 else 0.0


def _forced(m, z, q, d, u, T, pattern):
    tr = m.verify_sample_seq(z, q, d, u, T, force=dict(enumerate(pattern)))
    return tr.a, tr.c


def brute_outcomes(m, z, q, d, u, T, tol, grid=4001):
    """Outcomes reachable when near-tie decisions flip, by enumeration: every
    pattern of forced accept decisions whose deviations from the natural
    decision (from scipy's p) are all near ties, then every final uniform whose
    u*S moves by at most tol (grid over [-tol, tol])."""
    K = len(d)
    p = _p_rows(z, T)
    qq = np.asarray(q, np.float64)
    out = set()
    for pattern in itertools.product([False, True], repeat=K):
        a = next((k for k in range(K) if not pattern[k]), K)
        ok = True
        for k in range(min(a + 1, K)):
            r = _ratio(p[k], qq[k], int(d[k]))
            natural = np.float64(u[k]) < r
            if natural != pattern[k] and not (np.isfinite(r) and abs(np.float64(u[k]) - r) < tol):
                ok = False
        if not ok:
            continue
        mass = np.maximum(0.0, p[a] - qq[a]) if a < K else p[K]
        if a < K and not mass.sum() > 0.0:
            mass = p[a]
        S = mass.sum()
        for delta in np.linspace(-tol, tol, grid):
            uk = (np.float64(u[K]) * S + delta) / S
            if not (0.0 <= uk < 1.0):
                continue
            uu = np.array(u, np.float64)
            uu[K] = uk
            out.add(_forced(m, z, q, d, uu, T, pattern))
    return out


def _far_case(rng, V, K, T, margin=1e-3):
    """A random case whose decisions all lie at least `margin` from their
    thresholds (checked with scipy's p)."""
    while True:
        z, q = random_case(rng, V, K)
        d = [int(rng.integers(V)) for _ in range(K)]
        u = rng.random(K + 1)
        p = _p_rows(z, T)
        if any(abs(u[k] - _ratio(p[k], q[k], d[k])) < margin for k in range(K)):
            continue
        a = next((k for k in range(K) if not u[k] < _ratio(p[k], q[k], d[k])), K)
        mass = np.maximum(0.0, p[a] - q[a]) if a < K else p[K]
        if not mass.sum() > 0.0:
            continue
        cdf = np.cumsum(mass)
        if np.min(np.abs(cdf - u[K] * cdf[-1])) < margin:
            continue
        return z, q, d, u


def check_outcomes(m):
    """Failures of module m's sample_outcomes against the pins (empty = pass)."""
    fails = []
    rng = np.random.default_rng(71)
    T = 0.9
    # tol = 0: exactly the canonical outcome of verify_sample_seq, no flags
    for _ in range(40):
        z, q = random_case(rng, 5, 3)
        d = [int(rng.integers(5)) for _ in range(3)]
        u = rng.random(4)
        canon, allowed, flags = m.sample_outcomes(z, q, d, u, T, tol=0.0)
        tr = verify_sample_seq(z, q, d, u, T)
        if canon != (tr.a, tr.c) or allowed != [canon] or flags != 0:
            fails.append("tol=0 not exactly canonical")
            break
    # decisions far from every threshold: one outcome, no flags
    for _ in range(20):
        z, q, d, u = _far_case(rng, 5, 3, T)
        canon, allowed, flags = m.sample_outcomes(z, q, d, u, T, tol=1e-6)
        if allowed != [canon] or flags != 0:
            fails.append("far case widened")
            break
    # one accept test built 4e-7 from its threshold, either side: both the
    # continuation and the rejection are admitted, one flag
    K = 2
    for side in (-1.0, 1.0):
        z, q, d, u = _far_case(np.random.default_rng(72), 6, K, T)
        p = _p_rows(z, T)
        u = np.array(u, np.float64)
        u[0] = _ratio(p[0], q[0], d[0]) + side * 4e-7
        if not 0.0 <= u[0] < 1.0:
            fails.append("constructed tie out of range")
            continue
        want = {_forced(m, z, q, d, u, T, (True, u[1] < _ratio(p[1], q[1], d[1]))),
                _forced(m, z, q, d, u, T, (False, False))}
        canon, allowed, flags = m.sample_outcomes(z, q, d, u, T, tol=1e-6)
        if set(allowed) != want or flags != 1 or len(want) != 2:
            fails.append(f"accept near tie ({side:+.0f}): {allowed} vs {sorted(want)}, {flags} flags")
        # 4e-6 away it is no tie
        u[0] = _ratio(p[0], q[0], d[0]) + side * 4e-6
        canon, allowed, flags = m.sample_outcomes(z, q, d, u, T, tol=1e-6)
        if len(allowed) != 1 or flags != 0:
            fails.append("accept test 4e-6 away flagged")
    # two near ties in a row: three paths, two flags
    z, q, d, u = _far_case(np.random.default_rng(73), 6, K, T)
    p = _p_rows(z, T)
    u = np.array(u, np.float64)
    r0, r1 = _ratio(p[0], q[0], d[0]), _ratio(p[1], q[1], d[1])
    if r0 < 1.0 - 1e-5 and r1 < 1.0 - 1e-5:
        u[0], u[1] = r0 - 3e-7, r1 + 3e-7
        want = {_forced(m, z, q, d, u, T, pat) for pat in [(False, False), (True, False), (True, True)]}
        canon, allowed, flags = m.sample_outcomes(z, q, d, u, T, tol=1e-6)
        if set(allowed) != want or flags != 2:
            fails.append(f"two near ties: {allowed} vs {sorted(want)}, {flags} flags")
    else:
        fails.append("two-tie construction")
    # a bonus draw whose u*S sits 3e-7 past the boundary between tokens 1
    # and 2 of p_K: both neighbours, one flag; token 3 (zero mass) never
    zK = np.array([np.log(0.2), np.log(0.3), np.log(0.5), -np.inf, np.log(1e-300)])
    z = np.stack([zK, zK])
    q = softmax(zK)[None, :]                          # q = p: always accepted
    pK = softmax(zK)
    for eps, want in [(3e-7, {(1, 1), (1, 2)}), (-3e-7, {(1, 1), (1, 2)}), (3e-6, {(1, 2)}),
                      (-3e-6, {(1, 1)})]:
        u = np.array([0.5, (pK[0] + pK[1] + eps) / pK.sum()])
        canon, allowed, flags = m.sample_outcomes(z, q, [2], u, 1.0, tol=1e-6)
        if set(allowed) != want or flags != (len(want) > 1):
            fails.append(f"bonus boundary {eps}: {allowed}")
    # the residual draw after a rejection: boundary between two tokens with
    # positive residual, and a boundary whose neighbour has zero residual
    zr = np.log(np.array([0.3, 0.3, 0.2, 0.2]))
    q0 = np.array([0.1, 0.4, 0.1, 0.4])               # residual: 0.2, 0, 0.1, 0
    z = np.stack([zr, zr])
    r = np.maximum(0.0, softmax(zr) - q0)
    S = r.sum()
    for target, want in [(r[0] + 2e-7, {(0, 0), (0, 2)}), (r[0] - 2e-7, {(0, 0), (0, 2)}),
                         (r[0] + 5e-6, {(0, 2)})]:
        u = np.array([0.999, target / S])             # token 1: ratio 0.75, rejected
        canon, allowed, flags = m.sample_outcomes(z, q0[None, :], [1], u, 1.0, tol=1e-6)
        if set(allowed) != want:
            fails.append(f"residual boundary: {allowed} vs {want}")
    # brute force on tiny cases with a wide band (many ties at once), until
    # several cases with accept-test ties and several with draw ties are seen
    seen_accept = seen_draw = 0
    for seed in range(200):
        rr = np.random.default_rng(80 + seed)
        z, q = random_case(rr, 4, 2)
        d = [int(rr.integers(4)) for _ in range(2)]
        u = rr.random(3)
        tol = 0.1
        canon, allowed, flags = m.sample_outcomes(z, q, d, u, 1.0, tol=tol)
        brute = brute_outcomes(m, z, q, d, u, 1.0, tol, grid=801)
        if set(allowed) != brute:
            fails.append(f"brute force (seed {seed}): {allowed} vs {sorted(brute)}")
            break
        seen_accept += len({a for a, _ in brute}) > 1
        seen_draw += any(len({c for a2, c in brute if a2 == a}) > 1 for a, _ in brute)
        if seen_accept >= 5 and seen_draw >= 5:
            break
    else:
        fails.append(f"brute force saw too few ties ({seen_accept}, {seen_draw})")
    return fails


def test_sample_outcomes_pins():
    import oracle.verify as overify
    assert check_outcomes(overify) == []
