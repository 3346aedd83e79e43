"""Pins for the draft-tree verification oracle (oracle.tree).

* A chain (every node has one child) reduces to the chain verify oracles,
  which are pinned on their own: identical outcomes on random cases.
* Star trees (a root with m children drawn independently from q_0): the exact
  law of the first emitted token, measured by bisection over each uniform and
  weighted over every children tuple, equals scipy's softmax of the root row
  (the lossless property of rejection sampling, rskf.cn survey sections 1 and
  2.2) to 1e-12.
* Two-level trees whose target rows depend only on the token path: the first
  emitted token follows the root's softmax and the second, given the first,
  follows the softmax of that path's row (chi-square).
* Greedy: brute force over random trees with repeated sibling tokens.
* A hand example fixes the order in which siblings are tested.

``check_module`` holds the deterministic pins so planted mutants face them.
"""
import itertools

import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

import oracle.tree as otree
from oracle.verify import verify_greedy_seq, verify_sample_seq
from tests.pins import _steps, _threshold


def _random_tree(rng, N, V, width=3):
    parent = [0]
    for i in range(2, N + 1):
        parent.append(int(rng.integers(max(0, i - 1 - width), i)))
    token = rng.integers(0, V, size=N).tolist()
    return parent, token


def _star_law(m, z, q, T, V):
    """Exact law of the first emitted token of a star tree with m children."""
    parent = [0] * m
    law = np.zeros(V)
    for toks in itertools.product(range(V), repeat=m):
        w = float(np.prod([q[0, x] for x in toks]))
        if w == 0.0:
            continue

        def run(u):
            return otree.verify_tree_sample_seq(z, q, parent, list(toks), u, T)

        reach = 1.0
        u = [0.5] * (m + 1)
        for j in range(1, m + 1):
            def accepted(uj, j=j, base=list(u)):
                uu = list(base)
                uu[j] = uj
                a, _, nodes, _, _, _ = run(uu)
                return a >= 1 and nodes[0] == j
            t = _threshold(accepted)
            law[toks[j - 1]] += w * reach * t
            if t >= 1.0:
                reach = 0.0
                break
            reach *= 1.0 - t
            u[j] = 0.5 * (t + 1.0)              # reject child j from here on
        if reach > 0.0:
            def draw(u0, base=list(u)):
                uu = list(base)
                uu[0] = u0
                a, out, _, _, _, _ = run(uu)
                assert a == 0
                return int(out[0])
            for c, meas in _steps(draw).items():
                law[c] += w * reach * meas
    return law


def check_module(m):
    fails = []
    rng = np.random.default_rng(81)
    # chain reduction (sampled and greedy)
    for trial in range(60):
        K, V = int(rng.integers(1, 5)), int(rng.integers(2, 7))
        z = 2.0 * rng.standard_normal((K + 1, V))
        if trial % 5 == 0:
            z[rng.integers(K + 1), rng.integers(V)] = -np.inf
        q = softmax(z[:K] + rng.standard_normal((K, V)), axis=1)
        if trial % 7 == 0:
            q[:, rng.integers(V)] = 0.0
            q /= q.sum(axis=1, keepdims=True)
        d = [int(rng.choice(V, p=q[k])) for k in range(K)]
        u = rng.random(K + 1)
        tr = verify_sample_seq(z, q, d, u, 0.9)
        qt = np.vstack([q, np.full((1, V), 1.0 / V)])          # leaf row unused
        a, out, nodes, _, _, _ = m.verify_tree_sample_seq(z, qt, list(range(K)), d,
                                                           [u[K]] + list(u[:K]), 0.9)
        if a != tr.a or not np.array_equal(out, tr.out_tokens) or \
                list(nodes[:a]) != list(range(1, a + 1)):
            fails.append("chain sample")
            break
        ga, gc = verify_greedy_seq(z, d)
        a2, out2, _ = m.verify_tree_greedy_seq(z, list(range(K)), d)
        if a2 != ga or out2[a2] != gc:
            fails.append("chain greedy")
            break
    # greedy walk, brute force
    for _ in range(100):
        N, V = int(rng.integers(1, 9)), int(rng.integers(2, 5))
        parent, token = _random_tree(rng, N, V)
        z = rng.integers(-2, 3, size=(N + 1, V)).astype(np.float64)   # many ties
        a, out, nodes = m.verify_tree_greedy_seq(z, parent, token)
        cur = 0
        for j in range(a):
            n = int(nodes[j])
            g = min(v for v in range(V) if z[cur, v] == z[cur].max())
            kids = [i for i in range(1, N + 1) if parent[i - 1] == cur and token[i - 1] == g]
            if not kids or n != kids[0] or out[j] != g:
                fails.append("greedy walk")
                break
            cur = n
        g = min(v for v in range(V) if z[cur, v] == z[cur].max())
        if out[a] != g or any(parent[i - 1] == cur and token[i - 1] == g for i in range(1, N + 1)):
            fails.append("greedy stop")
        if np.any(out[a + 1:] != -1) or np.any(nodes[a:] != -1):
            fails.append("padding")
        if fails:
            break
    # sibling order: the lower-index child is tested first
    z = np.zeros((3, 2))
    q = np.full((3, 2), 0.5)
    a, out, nodes, _, _, _ = m.verify_tree_sample_seq(z, q, [0, 0], [0, 1], [0.9, 0.3, 0.3], 1.0)
    if not (a == 1 and nodes[0] == 1 and out[0] == 0):
        fails.append("sibling order")
    # star trees: exact law of the first token
    for mm, V, T in [(2, 3, 1.0), (3, 3, 0.7), (2, 4, 1.3)]:
        z = 2.0 * rng.standard_normal((mm + 1, V))
        q = softmax(rng.standard_normal((mm + 1, V)), axis=1)
        law = _star_law_m(m, mm, z, q, T, V)
        if np.abs(law - softmax(z[0] / T)).max() > 1e-12:
            fails.append(f"star law m={mm}")
    return fails


def _star_law_m(m, mm, z, q, T, V):
    saved = otree.verify_tree_sample_seq
    try:
        otree.verify_tree_sample_seq = m.verify_tree_sample_seq
        return _star_law(mm, z, q, T, V)
    finally:
        otree.verify_tree_sample_seq = saved


def test_oracle_passes_its_pins():
    assert check_module(otree) == []


def test_two_level_trees_follow_the_target():
    rng = np.random.default_rng(83)
    V, T, N_TRIALS = 4, 0.8, 20_000
    rows, qrows = {}, {}

    def row(path):
        if path not in rows:
            g = np.random.default_rng(abs(hash(path)) % (2 ** 32))
            rows[path] = 2.0 * g.standard_normal(V)
            qrows[path] = softmax(g.standard_normal(V))
        return rows[path], qrows[path]

    parent = [0, 0, 1, 1, 2, 2]                  # root -> 2 children -> 2 children each
    first = np.zeros(V, np.int64)
    second = {x: np.zeros(V, np.int64) for x in range(V)}
    for _ in range(N_TRIALS):
        tok, paths = [], {0: ()}
        for i in range(1, 7):
            _, qp = row(paths[parent[i - 1]])
            x = int(rng.choice(V, p=qp))
            tok.append(x)
            paths[i] = paths[parent[i - 1]] + (x,)
        z = np.stack([row(paths[n])[0] for n in range(7)])
        q = np.stack([row(paths[n])[1] for n in range(7)])
        a, out, _, _, _, _ = otree.verify_tree_sample_seq(z, q, parent, tok, rng.random(7), T)
        first[out[0]] += 1
        if a >= 1:
            second[out[0]][out[1]] += 1
    p0 = softmax(row(())[0] / T)
    assert stats.chisquare(first, p0 * N_TRIALS).pvalue > 1e-4
    for x in range(V):
        n = second[x].sum()
        if n > 2000:
            px = softmax(row((x,))[0] / T)
            assert stats.chisquare(second[x], px * n).pvalue > 1e-4, x


def test_outcomes_contain_the_result():
    rng = np.random.default_rng(85)
    for _ in range(50):
        N, V = int(rng.integers(1, 7)), int(rng.integers(2, 6))
        parent, token = _random_tree(rng, N, V)
        z = 2.0 * rng.standard_normal((N + 1, V))
        q = softmax(rng.standard_normal((N + 1, V)), axis=1)
        u = rng.random(N + 1)
        canon, allowed = otree.tree_outcomes(z, q, parent, token, u, 0.9)
        assert canon in allowed
        c0, a0 = otree.tree_outcomes(z, q, parent, token, u, 0.9, tol=0.0)
        assert a0 == [c0]
    # a test exactly at its threshold may go either way
    z = np.zeros((2, 2))
    q = np.array([[0.5, 0.5], [0.5, 0.5]])
    canon, allowed = otree.tree_outcomes(z, q, [0], [0], [0.25, 1.0 - 1e-9], 1.0)
    assert ((1,), 0) in allowed or ((1,), 1) in allowed
    assert any(p == () for p, _ in allowed)
