"""Checks that pin the oracle to facts outside itself.

The exact-law check treats a verify function as a black box f(d, u) -> (a, c):
it measures, by bisection over each uniform, how much of [0,1) leads to each
outcome, and weights draft tuples by the drafter's probabilities.  The result
is compared with the closed-form law of speculative sampling, which follows
from the lossless property (output distributed exactly as the target, rskf.cn
survey sections 1 and 2.2; Project 14, section 架构):

  P(out = [x_0..x_{a-1}, c]) = prod_{j<a} min(p_j(x_j), q_j(x_j))
                               * (max(0, p_a(c) - q_a(c))  if a < K
                                  p_K(c)                   if a = K)

with p_k = softmax(z_k / T) taken from scipy, q normalised.
"""
from __future__ import annotations

import itertools
from typing import Callable, Dict, Tuple

import numpy as np
from scipy.special import softmax

Outcome = Tuple[int, ...]  # (a, x_0..x_{a-1}, c)


def closed_form_law(z_rows: np.ndarray, q_rows: np.ndarray, T: float) -> Dict[Outcome, float]:
    K = q_rows.shape[0]
    V = z_rows.shape[1]
    p = [softmax(np.asarray(z_rows[k], dtype=np.float64) / T) for k in range(K + 1)]
    q = np.asarray(q_rows, dtype=np.float64)
    law: Dict[Outcome, float] = {}
    for a in range(K + 1):
        for prefix in itertools.product(range(V), repeat=a):
            w = 1.0
            for j, x in enumerate(prefix):
                w *= min(p[j][x], q[j][x])
            if w == 0.0:
                continue
            last = np.maximum(0.0, p[a] - q[a]) if a < K else p[K]
            for c in range(V):
                if last[c] > 0.0:
                    law[(a,) + prefix + (c,)] = law.get((a,) + prefix + (c,), 0.0) + w * last[c]
    return law


def _threshold(pred: Callable[[float], bool]) -> float:
    """sup{u in [0,1) : pred(u)} for a predicate true on [0, t) and false on [t, 1)."""
    grid = np.linspace(0.0, 1.0, 65)[:-1]
    vals = [pred(float(x)) for x in grid]
    # monotone check: once false, stays false
    first_false = next((i for i, v in enumerate(vals) if not v), None)
    if first_false is None:
        lo, hi = float(grid[-1]), 1.0
        if pred(np.nextafter(1.0, 0.0)):
            return 1.0
    else:
        assert not any(vals[first_false:]), "decision is not monotone in u"
        if first_false == 0:
            return 0.0
        lo, hi = float(grid[first_false - 1]), float(grid[first_false])
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if pred(mid):
            lo = mid
        else:
            hi = mid
    return hi


def _steps(f: Callable[[float], int]) -> Dict[int, float]:
    """Measure of {u in [0,1) : f(u) = c} for a non-decreasing step function f."""
    grid = list(np.linspace(0.0, 1.0, 65)[:-1]) + [float(np.nextafter(1.0, 0.0))]
    vals = [f(float(x)) for x in grid]
    breaks = []  # (position, value to the right)

    def rec(lo, hi, flo, fhi):
        if flo == fhi:
            return
        mid = 0.5 * (lo + hi)
        if hi - lo < 1e-15 or not (lo < mid < hi):
            breaks.append((hi, fhi))
            return
        fm = f(mid)
        rec(lo, mid, flo, fm)
        rec(mid, hi, fm, fhi)

    for i in range(len(grid) - 1):
        rec(grid[i], grid[i + 1], vals[i], vals[i + 1])
    meas: Dict[int, float] = {}
    pos, cur = 0.0, vals[0]
    for bpos, val in sorted(breaks):
        meas[cur] = meas.get(cur, 0.0) + (bpos - pos)
        pos, cur = bpos, val
    meas[cur] = meas.get(cur, 0.0) + (1.0 - pos)
    return meas


def blackbox_law(verify: Callable, z_rows: np.ndarray, q_rows: np.ndarray,
                 T: float) -> Dict[Outcome, float]:
    """Exact law of a verify function's outputs, found by bisection.

    ``verify(z_rows, q_rows, d, u, T)`` returns (a, c) for one sequence.
    """
    K = q_rows.shape[0]
    V = z_rows.shape[1]
    q = np.asarray(q_rows, dtype=np.float64)
    law: Dict[Outcome, float] = {}
    for d in itertools.product(range(V), repeat=K):
        wd = float(np.prod([q[k][d[k]] for k in range(K)]))
        if wd == 0.0:
            continue
        # acceptance threshold of each row, the earlier rows held at u = 0
        thr = []
        for k in range(K):
            def acc(uk, k=k):
                u = [0.0] * k + [uk] + [0.5] * (K - k)
                return verify(z_rows, q_rows, d, u, T)[0] > k
            thr.append(_threshold(acc))
        reach = 1.0
        for a in range(K + 1):
            if a < K:
                w = reach * (1.0 - thr[a])
            else:
                w = reach
            if w > 0.0:
                # force: rows < a accepted (u=0), row a rejected (u above its threshold)
                ua = [0.0] * a + ([0.5 * (thr[a] + 1.0)] if a < K else [])
                ua += [0.5] * (K - len(ua))

                def draw(uK, ua=ua):
                    res = verify(z_rows, q_rows, d, ua + [uK], T)
                    assert res[0] == a
                    return res[1]
                for c, m in _steps(draw).items():
                    if m > 0.0:
                        key = (a,) + tuple(d[:a]) + (c,)
                        law[key] = law.get(key, 0.0) + wd * w * m
            if a < K:
                reach *= thr[a]
    return law


def law_distance(l1: Dict[Outcome, float], l2: Dict[Outcome, float]) -> float:
    keys = set(l1) | set(l2)
    return max(abs(l1.get(k, 0.0) - l2.get(k, 0.0)) for k in keys)


def random_case(rng: np.random.Generator, V: int, K: int, zero_q: bool = False,
                neg_inf: bool = False):
    """Tiny verify case: logits [K+1, V], normalised draft probs [K, V]."""
    z = 2.0 * rng.standard_normal((K + 1, V))
    if neg_inf:
        z[0, rng.integers(V)] = -np.inf
    q = softmax(z[:K] + rng.standard_normal((K, V)), axis=1)
    if zero_q:
        q[:, rng.integers(V)] = 0.0
        q /= q.sum(axis=1, keepdims=True)
    return z, q
