"""Statistical pins for the oracle's sampled verify.

Fresh draft tokens d ~ q and uniforms u for N sequences that share one set of
target and draft rows.  The lossless property (rskf.cn survey sections 1 and
2.2; Project 14, section 架构) forces: the first emitted token ~ p_0, the token
after an accepted first draft ~ p_1, the bonus token (every draft accepted)
~ p_K.  Row k is accepted with probability beta_k = sum_v min(p_k, q_k), and
the mean accepted length is sum_{k=1..K} prod_{j<k} beta_j.  Chi-square (df =
V-1) and binomial / normal tests; thresholds p > 1e-4.
"""
import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

from oracle import verify_sample


def _chi2(counts, probs):
    n = counts.sum()
    keep = probs > 0
    assert counts[~keep].sum() == 0, "a zero-probability token was emitted"
    exp = probs[keep] * n
    # pool cells with small expectation into one
    small = exp < 5
    obs = counts[keep]
    if small.any():
        obs = np.concatenate([obs[~small], [obs[small].sum()]])
        exp = np.concatenate([exp[~small], [exp[small].sum()]])
    return stats.chisquare(obs, exp).pvalue


def _run(V, K, T, N, seed):
    rng = np.random.default_rng(seed)
    z = (2.0 * rng.standard_normal((K + 1, V))).astype(np.float32)
    q = softmax(z[:K].astype(np.float64) + rng.standard_normal((K, V)), axis=1)
    q32 = q.astype(np.float32)
    qn = q32.astype(np.float64) / q32.astype(np.float64).sum(axis=1, keepdims=True)
    d = np.stack([rng.choice(V, size=N, p=qn[k]) for k in range(K)], axis=1).astype(np.int32)
    u = rng.random((N, K + 1), dtype=np.float32)
    logits = np.broadcast_to(z, (N, K + 1, V))
    qs = np.broadcast_to(q32, (N, K, V))
    out, acc, _ = verify_sample(logits, "f32", qs, d, u, T)
    p = [softmax(z[k].astype(np.float64) / T) for k in range(K + 1)]
    beta = [np.minimum(p[k], q32[k].astype(np.float64)).sum() for k in range(K)]
    return out, acc, p, beta


@pytest.mark.parametrize("V,N", [(4, 200_000), (8, 200_000), (32, 100_000)])
def test_emitted_tokens_follow_target(V, N):
    K, T = 3, 1.0
    out, acc, p, beta = _run(V, K, T, N, seed=V)
    first = out[:, 0]
    assert _chi2(np.bincount(first, minlength=V), p[0]) > 1e-4
    second = out[acc >= 1, 1]
    assert _chi2(np.bincount(second, minlength=V), p[1]) > 1e-4
    bonus = out[acc == K, K]
    if bonus.size > 1000:
        assert _chi2(np.bincount(bonus, minlength=V), p[K]) > 1e-4
    # acceptance of row 0 ~ Binomial(N, beta_0)
    k0 = int((acc >= 1).sum())
    assert stats.binomtest(k0, N, beta[0]).pvalue > 1e-4
    # mean accepted length
    want = sum(np.prod(beta[:k]) for k in range(1, K + 1))
    se = acc.std() / np.sqrt(N)
    assert abs(acc.mean() - want) < 4.5 * se


def test_temperature_changes_target_not_draft():
    V, K, T, N = 6, 2, 0.5, 100_000
    out, acc, p, beta = _run(V, K, T, N, seed=77)
    assert _chi2(np.bincount(out[:, 0], minlength=V), p[0]) > 1e-4
    k0 = int((acc >= 1).sum())
    assert stats.binomtest(k0, N, beta[0]).pvalue > 1e-4
