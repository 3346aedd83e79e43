"""Pins for the mixed-batch verify oracle (oracle.mixed).

* A batch of sequences that share their logit and draft rows but carry
  different temperatures: within each temperature group the first emitted
  token follows scipy's softmax(z_0 / T) (chi-square), and the greedy group
  emits exactly numpy's argmax chain, whatever its uniforms.
* M2's invalid temperatures (negative, NaN, infinite, log2(e)/T overflowing fp32)
  verify greedily; the fp32 boundary of the overflow is checked directly.
* M3: p_draft of a greedy sequence is 1 exactly where the draft is the
  lowest-index argmax of its row, by brute force.
* A batch whose temperatures are all equal reduces to verify_sample, and an
  all-zero batch to verify_greedy (both pinned in their own files).

``check_module`` runs the deterministic pins on any module with the
oracle.mixed interface, so planted mutants face the same checks.
"""
import numpy as np
from scipy import stats
from scipy.special import softmax

import oracle.mixed as omixed
from oracle import verify_greedy, verify_sample


def _shared_batch(rng, N, K, V, temps):
    z = (2.0 * rng.standard_normal((K + 1, V))).astype(np.float32)
    q = softmax(z[:K].astype(np.float64) + rng.standard_normal((K, V)), axis=1).astype(np.float32)
    qn = q.astype(np.float64) / q.astype(np.float64).sum(axis=1, keepdims=True)
    d = np.stack([rng.choice(V, size=N, p=qn[k]) for k in range(K)], axis=1).astype(np.int32)
    u = rng.random((N, K + 1), dtype=np.float32)
    T = np.resize(np.asarray(temps, np.float32), N)
    return z, q, d, u, T


def _chi2(counts, probs):
    keep = probs > 0
    assert counts[~keep].sum() == 0
    exp = probs[keep] * counts.sum()
    small = exp < 5
    obs = counts[keep]
    if small.any():
        obs = np.concatenate([obs[~small], [obs[small].sum()]])
        exp = np.concatenate([exp[~small], [exp[small].sum()]])
    return stats.chisquare(obs, exp).pvalue


def check_module(m):
    fails = []
    rng = np.random.default_rng(61)
    # greedy group: exactly the argmax chain; mixed with sampled sequences
    K, V = 3, 6
    z, q, d, u, T = _shared_batch(rng, 60, K, V, [0.0, 0.7, 1.3])
    g = [int(np.argmax(z[k])) for k in range(K + 1)]
    d[0::3] = g[:K]                      # some greedy sequences accept everything
    d[3::6, 1] = (g[1] + 1) % V          # ... some reject at row 1
    out, acc, pd = m.verify_mixed(np.broadcast_to(z, (60, K + 1, V)), "f32",
                                  np.broadcast_to(q, (60, K, V)), d, u, T)
    for b in range(0, 60, 3):
        a = next((k for k in range(K) if d[b, k] != g[k]), K)
        want = np.full(K + 1, -1, np.int32)
        want[:a] = d[b, :a]
        want[a] = g[a]
        if acc[b] != a or not np.array_equal(out[b], want):
            fails.append("greedy chain")
            break
        wpd = np.array([1.0 if d[b, k] == g[k] else 0.0 for k in range(K)])
        if not np.array_equal(pd[b], wpd):
            fails.append("greedy p_draft")
            break
    # sampled sequences report p_k(d_k) at their own temperature
    for b in range(1, 60, 3):
        Tb = np.float64(T[b])
        wpd = np.array([softmax(z[k].astype(np.float64) / Tb)[d[b, k]] for k in range(K)])
        if not np.allclose(pd[b], wpd, rtol=1e-12):
            fails.append("sampled p_draft")
            break
    # invalid temperatures verify greedily
    # 3.5e-39 is invalid under M2 (log2(e)/T = 4.1e38 > FLT_MAX = 3.40e38)
    # although 1/T = 2.9e38 is finite; 4.5e-39 is valid (log2(e)/T = 3.2e38)
    bad = np.array([-1.0, np.nan, np.inf, 1e-39, 1e-38, 3.5e-39, 4.5e-39], dtype=np.float32)
    want_greedy = [True, True, True, True, False, True, False]
    nb = len(bad)
    zb = np.broadcast_to(z, (nb, K + 1, V))
    db = np.broadcast_to(np.array(g[:K], np.int32), (nb, K)).copy()
    db[:, 0] = (g[0] + 1) % V            # row 0 rejected by the greedy rule
    ub = np.full((nb, K + 1), 0.999, np.float32)
    outb, accb, _ = m.verify_mixed(zb, "f32", np.broadcast_to(q, (nb, K, V)), db, ub, bad)
    for i, wg in enumerate(want_greedy):
        if m.is_greedy(bad[i]) != wg:
            fails.append(f"is_greedy({bad[i]})")
        if wg and not (accb[i] == 0 and outb[i, 0] == g[0]):
            fails.append(f"invalid T={bad[i]} not greedy")
    if m.is_valid(np.float32(-1.0)) or not m.is_valid(np.float32(0.0)) or \
            not m.is_valid(np.float32(0.5)) or m.is_valid(np.float32(1e-39)):
        fails.append("is_valid")
    # reductions to the single-mode oracles
    z2 = (2.0 * rng.standard_normal((4, K + 1, V))).astype(np.float32)
    q2 = softmax(rng.standard_normal((4, K, V)), axis=2).astype(np.float32)
    d2 = rng.integers(0, V, size=(4, K)).astype(np.int32)
    u2 = rng.random((4, K + 1), dtype=np.float32)
    o1, a1, p1 = m.verify_mixed(z2, "f32", q2, d2, u2, np.full(4, 0.8, np.float32))
    o2, a2, p2 = verify_sample(z2, "f32", q2, d2, u2, float(np.float32(0.8)))
    if not (np.array_equal(o1, o2) and np.array_equal(a1, a2) and np.allclose(p1, p2, rtol=0)):
        fails.append("uniform temperature != verify_sample")
    o1, a1, _ = m.verify_mixed(z2, "f32", q2, d2, u2, np.zeros(4, np.float32))
    o2, a2 = verify_greedy(z2, "f32", d2)
    if not (np.array_equal(o1, o2) and np.array_equal(a1, a2)):
        fails.append("zero temperature != verify_greedy")
    return fails


def test_oracle_passes_its_pins():
    assert check_module(omixed) == []


def test_temperature_groups_follow_their_target():
    rng = np.random.default_rng(62)
    K, V, N = 2, 6, 60_000
    temps = [0.5, 1.5]
    z, q, d, u, T = _shared_batch(rng, N, K, V, temps)
    out, acc, _ = omixed.verify_mixed(np.broadcast_to(z, (N, K + 1, V)), "f32",
                                      np.broadcast_to(q, (N, K, V)), d, u, T)
    for Tg in temps:
        sel = T == np.float32(Tg)
        p0 = softmax(z[0].astype(np.float64) / np.float64(np.float32(Tg)))
        assert _chi2(np.bincount(out[sel, 0], minlength=V), p0) > 1e-4, Tg
    # the two groups really differ (a pin that ignores T would pass the above
    # only if both targets coincided)
    p_lo = softmax(z[0].astype(np.float64) / 0.5)
    p_hi = softmax(z[0].astype(np.float64) / 1.5)
    assert np.abs(p_lo - p_hi).max() > 0.05
