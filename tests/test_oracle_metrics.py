"""Pins for the acceptance-metrics oracle (oracle.metrics).

* A hand-counted example.
* Drafts accepted independently with probability alpha (accept count
  min(Geometric, K)): the acceptance length tends to sum_{k=1..K} alpha^k and
  every conditional rate to alpha (closed forms of the truncated geometric).
* Driven by the verify oracle: q = p accepts every draft (acceptance length
  K, rate 1); a one-hot q on a zero of p rejects every first draft (0, 0).
* Counters over several calls add up to the counters of the concatenation.
"""
import numpy as np
import pytest
from scipy.special import softmax

import oracle.metrics as ometrics
from oracle import verify_sample


def check_module(m):
    fails = []
    c = m.counters([0, 3, 3, 1], 3)
    r = m.rates(c)
    if not (c["rounds"] == 4 and c["proposed"] == 12 and c["accepted"] == 7 and c["emitted"] == 11
            and list(c["hist"]) == [1, 1, 0, 2]):
        fails.append("hand counters")
    if not (r["acceptance_length"] == 1.75 and r["tokens_per_round"] == 2.75
            and r["draft_acceptance_rate"] == 7 / 12
            and np.allclose(r["conditional_rate"], [0.75, 2 / 3, 1.0])):
        fails.append("hand rates")
    parts = [[0, 1, 2], [2, 2], [0]]
    tot = m.counters(parts[0], 2)
    for p in parts[1:]:
        tot = m.accumulate(tot, m.counters(p, 2))
    whole = m.counters(sum(parts, []), 2)
    if not (tot["steps"] == 3 and all(np.array_equal(tot[k], whole[k])
                                      for k in ("rounds", "proposed", "accepted", "emitted", "hist"))):
        fails.append("accumulate")
    return fails


def test_oracle_passes_its_pins():
    assert check_module(ometrics) == []


@pytest.mark.parametrize("alpha,K", [(0.76, 5), (0.5, 7), (0.9, 3)])
def test_independent_acceptance_closed_form(alpha, K):
    rng = np.random.default_rng(int(alpha * 100) + K)
    N = 200_000
    a = np.minimum(rng.geometric(1 - alpha, size=N) - 1, K)     # accepted before the first reject
    r = ometrics.rates(ometrics.counters(a, K))
    want = sum(alpha ** k for k in range(1, K + 1))
    assert abs(r["acceptance_length"] - want) < 5 * a.std() / np.sqrt(N)
    assert abs(r["tokens_per_round"] - (want + 1)) < 5 * a.std() / np.sqrt(N)
    assert np.allclose(r["conditional_rate"], alpha, atol=0.01)


def test_driven_by_the_verify_oracle():
    rng = np.random.default_rng(3)
    B, K, V = 50, 4, 12
    z = (2.0 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    p = softmax(z[:, :K].astype(np.float64), axis=2).astype(np.float32)
    pn = p.astype(np.float64)
    pn /= pn.sum(axis=2, keepdims=True)
    d = np.stack([[rng.choice(V, p=pn[b, k]) for k in range(K)] for b in range(B)]).astype(np.int32)
    u = rng.random((B, K + 1), dtype=np.float32)
    _, acc, _ = verify_sample(z, "f32", p, d, u, 1.0)
    r = ometrics.rates(ometrics.counters(acc, K))
    assert r["acceptance_length"] == K and r["draft_acceptance_rate"] == 1.0
    # one-hot q on a token the target never emits
    z2 = z.copy()
    z2[:, :, 0] = -np.inf
    q = np.zeros((B, K, V), np.float32)
    q[:, :, 0] = 1.0
    d0 = np.zeros((B, K), np.int32)
    _, acc0, _ = verify_sample(z2, "f32", q, d0, u, 1.0)
    r0 = ometrics.rates(ometrics.counters(acc0, K))
    assert r0["acceptance_length"] == 0 and r0["draft_acceptance_rate"] == 0.0
    assert r0["conditional_rate"][0] == 0.0 and np.isnan(r0["conditional_rate"][1])
