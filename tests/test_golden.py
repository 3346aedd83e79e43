"""Checks against numbers the pages print.

usage_log_decode.json: the sample session of Project 14 logs 3.2 accepted
tokens per step at an acceptance rate of 0.76.  With i.i.d. acceptance alpha
per draft, a step emits sum_{k=0..K} alpha^k tokens on average (the accepted
drafts plus the resampled or bonus token).  The oracle, run on rows whose
per-draft acceptance is exactly 0.76, must reproduce that closed form, and
3.2 must fall between its values at K = 4 and K = 5 (it exceeds the K -> inf
limit of alpha/(1-alpha) = 3.17 accepted drafts without the extra token, so
the log counts the emitted token too).

peagle_serve_config.json: K = 7 drafts and 1024 concurrent sequences; the
draft batch the oracle builds must hold K-1 MASK rows per sequence and fit the
verify batch plus the K x max_num_seqs capture extension.
"""
import json
import os

import numpy as np

from oracle import build_draft_batch, verify_sample

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def test_usage_log_acceptance_closed_form():
    g = _load("usage_log_decode.json")
    alpha, per_step = g["acceptance_rate"], g["accepted_tokens_per_step"]
    closed = {K: sum(alpha ** k for k in range(K + 1)) for K in (4, 5)}
    assert closed[4] < per_step < closed[5]
    assert alpha / (1 - alpha) < per_step
    # rows with sum_v min(p, q) = 0.5 + 0.26 = 0.76 exactly
    z_row = np.array([0.0, 0.0], dtype=np.float32)
    q_row = np.array([0.74, 0.26])
    rng = np.random.default_rng(2026)
    for K in (4, 5):
        N = 40_000
        logits = np.broadcast_to(z_row, (N, K + 1, 2))
        qs = np.broadcast_to(q_row, (N, K, 2))
        d = (rng.random((N, K)) >= 0.74).astype(np.int32)          # d ~ q
        u = rng.random((N, K + 1))
        _, acc, _ = verify_sample(logits, "f32", qs, d, u, 1.0)
        emitted = acc + 1
        se = emitted.std() / np.sqrt(N)
        assert abs(emitted.mean() - closed[K]) < 4.5 * se
        tested = np.minimum(acc + 1, K).sum()
        assert abs(acc.sum() / tested - alpha) < 0.01


def test_serve_config_draft_batch_shape():
    g = _load("peagle_serve_config.json")
    K, S = g["num_speculative_tokens"], g["max_num_seqs"]
    rows_per_seq = 2 * K
    assert S * rows_per_seq <= S * (K + 1) + K * S
    # a few sequences of that shape through the oracle: K-1 MASK rows each
    B, H, bs = 4, 8, 16
    rng = np.random.default_rng(7)
    a = np.array([0, 3, 7, 5], dtype=np.int32)
    d = rng.integers(0, 1000, size=(B, K)).astype(np.int32)
    out = np.full((B, K + 1), -1, dtype=np.int32)
    for b in range(B):
        out[b, :a[b]] = d[b, :a[b]]
        out[b, a[b]] = 999
    L = np.array([5, 100, 17, 64], dtype=np.int64)
    bt = np.arange(B * 8, dtype=np.int32).reshape(B, 8)
    res = build_draft_batch(out, a, d, L, bt, bs, np.zeros((B * (K + 1), H), np.uint16),
                            np.ones(H, np.uint16), 5000)
    assert res["input_ids"].shape == (B * rows_per_seq,)
    for b in range(B):
        seg = res["input_ids"][b * 2 * K:(b + 1) * 2 * K]
        assert int((seg == 5000).sum()) == K - 1
