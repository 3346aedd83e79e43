"""Oracle: one verify batch whose sequences carry their own temperature.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

A serving batch gathers requests from many clients ("Project 14 -
speculative decoding inference server", section 架构: request ingress into
one vLLM / SGLang server that verifies every running sequence's drafts in a
single target pass), and each request brings its own sampling settings.
Section 概念 of the same page describes the greedy case (an accepted prefix
replaces the greedy path); the sampled case is the rejection sampling of
``verify.verify_sample_seq``.

Readings (the pages give no per-request interface):

* M1  temperatures[b] = 0 selects the greedy rule for sequence b
      (``verify.verify_greedy_seq``); temperatures[b] > 0 selects rejection
      sampling at that temperature (``verify.verify_sample_seq``).  Draft
      probabilities and uniforms of greedy sequences are not used.
* M2  a temperature that is negative, NaN or infinite is invalid, and so is
      one so small that the exponent scale log2(e)/T, the factor with which
      softmax(z/T) is evaluated as powers of two, is not a finite fp32
      number (T below about 4.24e-39, a subnormal): that sequence is verified
      greedily and flagged.  The pages fix no lower limit; this one is the
      point below which z/T cannot be formed in fp32 at all.
* M3  p_draft of a greedy sequence is the T -> 0 limit of p_k(d_k): 1 where
      d_k is row k's lowest-index argmax, else 0.
"""
from __future__ import annotations

import numpy as np

from .verify import assemble, decode_logits, first_argmax, verify_greedy_seq, verify_sample_seq

LOG2E = 1.4426950408889634


def is_greedy(T: float) -> bool:
    """M1/M2: does a sequence with temperature T (an fp32 value) verify greedily?"""
    T32 = np.float32(T)
    if T32 == 0.0:
        return True
    if not (T32 > 0.0 and np.isfinite(T32)):
        return True                         # invalid (M2)
    with np.errstate(over="ignore"):
        c = np.float32(LOG2E / np.float64(T32))
    return not np.isfinite(c)               # log2(e)/T overflows fp32 (M2)


def is_valid(T: float) -> bool:
    """False for the temperatures M2 flags."""
    T32 = np.float32(T)
    return bool(T32 == 0.0 or not is_greedy(T32))


def verify_mixed_seq(z_rows: np.ndarray, q_rows: np.ndarray, d, u, T: float):
    """(a, out_tokens row, p_draft row) of one sequence under M1-M3."""
    K = len(d)
    if is_greedy(T):
        a, c = verify_greedy_seq(z_rows, d)
        pd = np.array([1.0 if int(d[k]) == first_argmax(z_rows[k]) else 0.0 for k in range(K)])
        return a, assemble(d, a, c), pd
    tr = verify_sample_seq(z_rows, q_rows, d, u, float(np.float32(T)))
    return tr.a, tr.out_tokens, tr.p_draft


def verify_mixed(logits: np.ndarray, dtype: str, draft_probs: np.ndarray,
                 draft_tokens: np.ndarray, uniforms: np.ndarray, temperatures: np.ndarray):
    """Batch verify with per-sequence temperatures (fp32 [B]).

    Returns (out_tokens [B,K+1] int32, num_accepted [B] int32, p_draft [B,K] fp64).
    """
    B, K1, V = logits.shape
    K = K1 - 1
    out = np.empty((B, K + 1), dtype=np.int32)
    acc = np.empty(B, dtype=np.int32)
    pd = np.empty((B, K), dtype=np.float64)
    for b in range(B):
        a, out[b], pd[b] = verify_mixed_seq(decode_logits(logits[b], dtype), draft_probs[b],
                                            draft_tokens[b], uniforms[b], temperatures[b])
        acc[b] = a
    return out, acc, pd
