"""Pins for the drafter-output sampling oracle (oracle.draft).

What fixes it from outside:
* q for T > 0 is the softmax at temperature T: scipy.special.softmax(z / T);
* T = 0 (greedy drafting) gives a one-hot q at the lowest-index maximum, found
  here by brute force over the row;
* the draw is the inverse CDF: numpy.searchsorted over the cumulative sum, and
  the midpoint of every token's CDF cell returns that token;
* drawn tokens follow q (chi-square);
* end to end, drafting with it and verifying with the verify oracle emits a
  first token distributed as the target softmax, row 0 is accepted with
  probability sum_v min(p_0, q_0), and the mean accepted length is
  sum_{k=1..K} prod_{j<k} beta_j (the lossless property of speculative
  sampling, rskf.cn survey sections 1 and 2.2; Project 14, section 架构).

``check_module`` runs the deterministic pins against any module with the
oracle.draft interface, so planted mutants can be checked with the same code.
"""
import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

import oracle.draft as odraft
from oracle import verify_sample


def _rows_case(rng, V, with_inf=False, ties=False):
    z = (2.0 * rng.standard_normal(V)).astype(np.float32)
    if with_inf:
        z[rng.choice(V, size=max(1, V // 4), replace=False)] = -np.inf
    if ties:
        m = z.max()
        z[rng.choice(V, size=2, replace=False)] = m + 1.0
    return z


def check_module(m):
    """Failures of ``m`` against the deterministic pins (empty list: all pass)."""
    fails = []
    rng = np.random.default_rng(31)
    # softmax at temperature T
    for T in (0.5, 0.7, 1.0, 1.3):
        for V in (2, 7, 33):
            z = _rows_case(rng, V, with_inf=(V > 2))
            q = m.draft_distribution(z.astype(np.float64), T)
            want = softmax(z.astype(np.float64) / T)
            if not np.allclose(q, want, rtol=1e-13, atol=1e-300):
                fails.append(f"softmax T={T} V={V}")
    # greedy: one-hot at the lowest maximum
    for V in (3, 9, 40):
        z = _rows_case(rng, V, ties=True)
        lowest = min(i for i in range(V) if z[i] == z.max())
        q = m.draft_distribution(z.astype(np.float64), 0.0)
        d, q2 = m.draft_sample_row(z.astype(np.float64), 0.0, 0.9)
        if not (q[lowest] == 1.0 and q.sum() == 1.0 and d == lowest and np.array_equal(q, q2)):
            fails.append(f"greedy V={V}")
    # inverse CDF: searchsorted, and cell midpoints
    for _ in range(200):
        V = int(rng.integers(2, 30))
        z = _rows_case(rng, V, with_inf=bool(rng.random() < 0.5))
        T = float(rng.choice([0.6, 1.0, 1.4]))
        u = float(rng.random(dtype=np.float32))
        d, q = m.draft_sample_row(z.astype(np.float64), T, u)
        cdf = np.cumsum(q)
        want = int(np.searchsorted(cdf, u * cdf[-1], side="right"))
        if d != want or q[d] <= 0.0:
            fails.append("searchsorted")
            break
        lo = np.concatenate([[0.0], cdf[:-1]])
        for v in np.nonzero(q > 0)[0]:
            mid = 0.5 * (lo[v] + cdf[v]) / cdf[-1]
            if m.draft_sample_row(z.astype(np.float64), T, mid)[0] != v:
                fails.append("cell midpoint")
                break
    # batch API: explicit gather and per-sequence temperatures, brute force
    B, K, V, R = 4, 3, 12, 20
    logits = (2.0 * rng.standard_normal((R, V))).astype(np.float32)
    u = rng.random((B, K), dtype=np.float32)
    rows = rng.choice(R, size=B * K, replace=False).astype(np.int32).reshape(B, K)
    temps = np.array([0.0, 0.5, 1.0, 1.3], dtype=np.float32)
    d, q = m.draft_sample(logits, "f32", u, 0.8, B, K, row_index=rows, temperatures=temps)
    for b in range(B):
        for k in range(K):
            zb = logits[rows[b, k]].astype(np.float64)
            Tb = float(temps[b])
            if Tb == 0.0:
                wq = np.zeros(V); wq[int(np.argmax(zb))] = 1.0
                wd = int(np.argmax(zb))
            else:
                wq = softmax(zb / Tb)
                c = np.cumsum(wq)
                wd = int(np.searchsorted(c, np.float64(u[b, k]) * c[-1], side="right"))
            if d[b, k] != wd or not np.allclose(q[b, k], wq, rtol=1e-13, atol=0):
                fails.append("batch gather / temperatures")
                break
    d2, q2 = m.draft_sample(logits[: B * K], "f32", u, 0.8, B, K)
    for b in range(B):
        for k in range(K):
            wd, wq = odraft.draft_sample_row(logits[b * K + k].astype(np.float64), np.float32(0.8),
                                             u[b, k])
            if d2[b, k] != wd:
                fails.append("default rows")
                break
    return fails


def test_oracle_passes_its_pins():
    assert check_module(odraft) == []


def test_temperature_and_scalar_precision():
    # the scalar temperature is an fp32 value widened to fp64, as it is passed
    z = np.array([0.0, 1.0, 3.0])
    d, q = odraft.draft_sample(z[None, :].astype(np.float32), "f32",
                               np.array([[0.5]], np.float32), 0.7, 1, 1)
    assert np.allclose(q[0, 0], softmax(z / np.float64(np.float32(0.7))), rtol=1e-15)
    with pytest.raises(ValueError):
        odraft.draft_distribution(z, -1.0)
    with pytest.raises(ValueError):
        odraft.draft_distribution(z, float("nan"))


def test_bf16_rows_decode_exactly():
    bits = np.array([[0x3F80, 0x4000, 0xFF80, 0x4040]], dtype=np.uint16)  # 1, 2, -inf, 3
    d, q = odraft.draft_sample(bits, "bf16", np.array([[0.0]], np.float32), 1.0, 1, 1)
    assert np.allclose(q[0, 0], softmax(np.array([1.0, 2.0, -np.inf, 3.0])), rtol=1e-15)
    assert d[0, 0] == 0            # u = 0 takes the first positive-mass token
    assert q[0, 0, 2] == 0.0


def test_outcomes_contain_the_draw():
    rng = np.random.default_rng(5)
    for _ in range(100):
        V = int(rng.integers(2, 20))
        z = _rows_case(rng, V)
        u = float(rng.random(dtype=np.float32))
        d, q = odraft.draft_sample_row(z.astype(np.float64), 0.9, u)
        assert odraft.draft_outcomes(z, 0.9, u, tol=0.0) == [d]
        assert d in odraft.draft_outcomes(z, 0.9, u)
    # u*S exactly on a boundary: both neighbours are acceptable within tol
    z = np.log(np.array([0.25, 0.25, 0.5]))
    assert odraft.draft_outcomes(z, 1.0, 0.25) == [0, 1]
    assert odraft.draft_outcomes(z, 0.0, 0.25) == [2]


def _chi2(counts, probs):
    keep = probs > 0
    assert counts[~keep].sum() == 0, "a zero-probability token was drawn"
    exp = probs[keep] * counts.sum()
    return stats.chisquare(counts[keep], exp).pvalue


def test_draws_follow_q():
    rng = np.random.default_rng(41)
    V, N, T = 8, 40_000, 0.8
    z = (2.0 * rng.standard_normal(V)).astype(np.float32)
    z[3] = -np.inf
    logits = np.broadcast_to(z, (N, V))
    u = rng.random((N, 1), dtype=np.float32)
    d, q = odraft.draft_sample(logits, "f32", u, T, N, 1)
    assert _chi2(np.bincount(d[:, 0], minlength=V), q[0, 0]) > 1e-4


def test_end_to_end_drafting_then_verify_is_lossless():
    """Drafts sampled by the oracle, verified by the verify oracle: the emitted
    tokens follow the target, acceptance follows beta = sum min(p, q)."""
    rng = np.random.default_rng(43)
    V, K, T, N = 6, 3, 0.9, 40_000
    zt = (2.0 * rng.standard_normal((K + 1, V))).astype(np.float32)      # target rows
    zd = (zt[:K] + rng.standard_normal((K, V))).astype(np.float32)         # drafter rows
    du = rng.random((N, K), dtype=np.float32)
    d, q = odraft.draft_sample(np.tile(zd, (N, 1)), "f32", du, T, N, K)
    q32 = q.astype(np.float32)
    vu = rng.random((N, K + 1), dtype=np.float32)
    out, acc, _ = verify_sample(np.broadcast_to(zt, (N, K + 1, V)), "f32", q32, d, vu, T)
    p = [softmax(zt[k].astype(np.float64) / T) for k in range(K + 1)]
    qk = [softmax(zd[k].astype(np.float64) / T) for k in range(K)]
    beta = [np.minimum(p[k], qk[k]).sum() for k in range(K)]
    assert _chi2(np.bincount(out[:, 0], minlength=V), p[0]) > 1e-4
    assert stats.binomtest(int((acc >= 1).sum()), N, beta[0]).pvalue > 1e-4
    want = sum(np.prod(beta[:k]) for k in range(1, K + 1))
    assert abs(acc.mean() - want) < 4.5 * acc.std() / np.sqrt(N)
