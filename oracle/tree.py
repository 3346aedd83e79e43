"""Oracle: verification of a draft tree, fp64, one sequence at a time.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

"Project 14 - speculative decoding inference server", section 概念, says that
P-EAGLE's parallel speculation forms deeper draft trees; the pages give no
tree shape and no tree acceptance rule.  The readings below are the plainest
ones that keep the method's defining property (the emitted tokens follow the
target, rskf.cn survey sections 1 and 2.2) and reduce to the chain verify of
``verify`` when every node has one child.

Tree.  N draft nodes 1..N; node 0 is the root (the last committed token).
parent[i] < i names node i's parent (nodes are in topological order),
token[i] its token.  Target logit row n (n = 0..N) is the target's
distribution after node n; draft-probability row n is the drafter
distribution from which node n's children were drawn, independently.
Uniforms: u[i] (i = 1..N) decides node i's test, u[0] drives the final draw.

* T1 greedy: from the root, move to the lowest-index child whose token is the
     argmax g of the current row (lowest index, as R7); when no child matches,
     emit g.  The path's tokens and g are emitted.
* T2 sampled: at the current node, with r = p (the target row at T), test its
     children in index order: child x is accepted iff u < r(x) / q(x) (q(x) = 0:
     accepted iff r(x) > 0).  On a rejection r becomes max(0, r - q)
     normalised (if that is all zero, r becomes p: only reachable by
     rounding).  An accepted child becomes the current node; when every child
     is rejected, or the node is a leaf, the new token is drawn from r by the
     inverse CDF with u[0].  This is recursive rejection sampling over
     independently drafted candidates.
* T3 outputs: out_tokens = path tokens, the new token, then -1 up to N+1
     entries; out_path = the accepted node indices, then -1; a = path length.
"""
from __future__ import annotations

from typing import List, Optional, Sequence, Tuple

import numpy as np

from .verify import _draw_candidates, first_argmax, inverse_cdf, target_distribution


def children(parent: Sequence[int], n: int) -> List[int]:
    """Child nodes of node n in index order."""
    return [i for i in range(1, len(parent) + 1) if int(parent[i - 1]) == n]


def check_tree(parent: Sequence[int], token: Sequence[int], V: int) -> None:
    for i in range(1, len(parent) + 1):
        assert 0 <= int(parent[i - 1]) < i, f"node {i}: parent must precede it"
        assert 0 <= int(token[i - 1]) < V, f"node {i}: token outside the vocabulary"


def _assemble(N: int, path: List[int], token: Sequence[int], c: int):
    out = np.full(N + 1, -1, dtype=np.int32)
    nodes = np.full(N + 1, -1, dtype=np.int32)
    for j, n in enumerate(path):
        out[j] = int(token[n - 1])
        nodes[j] = n
    out[len(path)] = c
    return out, nodes


def verify_tree_greedy_seq(z_rows: np.ndarray, parent, token):
    """T1.  Returns (a, out_tokens [N+1], out_path [N+1])."""
    N = len(parent)
    check_tree(parent, token, z_rows.shape[1])
    cur, path = 0, []
    while True:
        g = first_argmax(z_rows[cur])
        nxt = next((i for i in children(parent, cur) if int(token[i - 1]) == g), None)
        if nxt is None:
            out, nodes = _assemble(N, path, token, g)
            return len(path), out, nodes
        path.append(nxt)
        cur = nxt


def verify_tree_sample_seq(z_rows: np.ndarray, q_rows: np.ndarray, parent, token,
                           u: Sequence[float], T: float, force: Optional[dict] = None):
    """T2.  Returns (a, out_tokens [N+1], out_path [N+1], draw mass, u[0], tests)
    where tests lists (node, ratio) for every test made.  The draw mass is p
    when no child of the last node was rejected, else the last unnormalised
    residual max(0, r - q) (the inverse CDF is unchanged by normalisation;
    this keeps the one-child case identical to the chain verify).

    ``force`` (test use) maps node i -> bool to override its test."""
    N = len(parent)
    check_tree(parent, token, z_rows.shape[1])
    q = np.asarray(q_rows, dtype=np.float64)
    cur, path, tests = 0, [], []
    while True:
        p = target_distribution(z_rows[cur], T)
        r, mass = p, p
        nxt = None
        for i in children(parent, cur):
            x = int(token[i - 1])
            if q[cur, x] > 0.0:
                ratio = r[x] / q[cur, x]
            else:
                ratio = np.inf if r[x] > 0.0 else 0.0
            tests.append((i, ratio))
            ok = np.float64(u[i]) < ratio
            if force is not None and i in force:
                ok = bool(force[i])
            if ok:
                nxt = i
                break
            res = np.maximum(0.0, r - q[cur])
            S = res.sum()
            if S > 0.0:
                r, mass = res / S, res
            else:
                r, mass = p, p
        if nxt is None:
            c, _, _ = inverse_cdf(mass, float(u[0]))
            out, nodes = _assemble(N, path, token, c)
            return len(path), out, nodes, mass, float(u[0]), tests
        path.append(nxt)
        cur = nxt


def verify_tree(logits64: np.ndarray, parents: np.ndarray, tokens: np.ndarray,
                draft_probs: Optional[np.ndarray] = None, uniforms: Optional[np.ndarray] = None,
                T: float = 0.0):
    """Batch: logits64 [B][N+1][V] fp64 (decoded), parents / tokens [B][N].
    T = 0: greedy (T1); T > 0: sampled (T2).
    Returns (out_tokens [B][N+1], out_path [B][N+1], num_accepted [B])."""
    B, N1, V = logits64.shape
    out = np.empty((B, N1), np.int32)
    nodes = np.empty((B, N1), np.int32)
    acc = np.empty(B, np.int32)
    for b in range(B):
        if T == 0.0:
            a, o, n = verify_tree_greedy_seq(logits64[b], parents[b], tokens[b])
        else:
            a, o, n, _, _, _ = verify_tree_sample_seq(logits64[b], draft_probs[b], parents[b],
                                                      tokens[b], uniforms[b], T)
        out[b], nodes[b], acc[b] = o, n, a
    return out, nodes, acc


def tree_outcomes(z_rows, q_rows, parent, token, u, T, tol: float = 1e-6):
    """Outcomes (path tuple, new token) an evaluation exact up to ``tol`` may
    return: a test whose u lies within tol of its ratio may go either way
    (replayed with that decision forced), and the final draw may return any
    token whose CDF cell lies within tol of u*S.  Returns (canonical, allowed)."""
    a, out, nodes, _, _, _ = verify_tree_sample_seq(z_rows, q_rows, parent, token, u, T)
    canon = (tuple(int(x) for x in nodes[:a]), int(out[a]))
    allowed = set()
    seen = set()

    def walk(force):
        key = tuple(sorted(force.items()))
        if key in seen:
            return
        seen.add(key)
        a2, _, nodes2, mass, u0, tests = verify_tree_sample_seq(z_rows, q_rows, parent, token,
                                                                 u, T, force=force)
        path = tuple(int(x) for x in nodes2[:a2])
        for c in _draw_candidates(mass, u0, tol):
            allowed.add((path, c))
        for i, ratio in tests:
            if i not in force and abs(float(u[i]) - ratio) < tol:
                f2 = dict(force)
                f2[i] = not (np.float64(u[i]) < ratio)
                walk(f2)

    walk({})
    return canon, sorted(allowed)
