"""Pins for the oracle's greedy verify.

The fact pinned: with greedy decoding the emitted tokens are exactly the
target's greedy continuation (Project 14, section 概念: the accepted prefix
replaces the greedy path; rskf.cn survey section 2.2: the output equals plain
autoregressive decoding).  Per sequence that means: the drafts are kept up to
the first one that differs from the target argmax of its row, and the next
emitted token is that row's argmax.  The checks use numpy's argmax and brute
force over all draft tuples of tiny vocabularies.
"""
import itertools

import numpy as np
import pytest

from oracle import verify_greedy
from oracle.verify import verify_greedy_seq


def _greedy_chain_property(z, d, a, c):
    """a and c are what the greedy-continuation property forces."""
    K = len(d)
    g = [int(np.argmax(z[k])) for k in range(K + 1)]
    agree = 0
    while agree < K and d[agree] == g[agree]:
        agree += 1
    return a == agree and c == g[agree]


@pytest.mark.parametrize("V,K", [(2, 1), (3, 2), (4, 3)])
def test_all_draft_tuples_tiny(V, K):
    rng = np.random.default_rng(V * 10 + K)
    for _ in range(5):
        z = rng.integers(-2, 3, size=(K + 1, V)).astype(np.float64)  # many ties
        for d in itertools.product(range(V), repeat=K):
            a, c = verify_greedy_seq(z, list(d))
            assert _greedy_chain_property(z, d, a, c)


def test_batch_shapes_and_padding():
    rng = np.random.default_rng(7)
    B, K, V = 16, 5, 50
    z = rng.standard_normal((B, K + 1, V)).astype(np.float32)
    g = z.argmax(axis=2)
    d = g[:, :K].copy().astype(np.int32)
    # sequence b keeps b % (K+1) drafts: corrupt draft a_b when a_b < K
    want_a = np.arange(B) % (K + 1)
    for b in range(B):
        if want_a[b] < K:
            d[b, want_a[b]] = (g[b, want_a[b]] + 1) % V
    out, acc = verify_greedy(z, "f32", d)
    assert np.array_equal(acc, want_a)
    for b in range(B):
        a = want_a[b]
        assert np.array_equal(out[b, :a], d[b, :a])
        assert out[b, a] == g[b, a]
        assert np.all(out[b, a + 1:] == -1)


def test_special_cases():
    z = np.array([[0.0, 1.0, 0.5], [2.0, 0.0, 0.0], [0.0, 0.0, 3.0]])
    # every draft is the argmax -> a = K and the bonus is the last row's argmax
    assert verify_greedy_seq(z, [1, 0]) == (2, 2)
    # first draft wrong -> a = 0, c = argmax of row 0
    assert verify_greedy_seq(z, [2, 0]) == (0, 1)
    # tie in row 0 between tokens 1 and 2: the lowest index is the argmax
    zt = np.array([[0.0, 1.0, 1.0], [0.0, 0.0, 1.0]])
    assert verify_greedy_seq(zt, [2]) == (0, 1)
    assert verify_greedy_seq(zt, [1]) == (1, 2)


def test_bf16_batch_matches_property():
    rng = np.random.default_rng(11)
    B, K, V = 8, 7, 300
    bits = rng.integers(0x3C00, 0x4100, size=(B, K + 1, V)).astype(np.uint16)  # many ties
    z = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    d = np.where(rng.random((B, K)) < 0.7, z[:, :K].argmax(axis=2),
                 rng.integers(0, V, size=(B, K))).astype(np.int32)
    out, acc = verify_greedy(bits, "bf16", d)
    for b in range(B):
        assert _greedy_chain_property(z[b], list(d[b]), int(acc[b]), int(out[b, acc[b]]))
