"""Oracle: sampling the drafter's prediction rows into the next verify's draft
tokens and draft probabilities, fp64, one row at a time.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

After the P-EAGLE drafter's single forward over the batch that the build made,
each sequence has K prediction rows: the NTP row and the K-1 MASK rows, which
together predict all K drafts in parallel (P-EAGLE / TorchSpec blog summary,
the section on parallel drafting; the build lists those rows as sample_rows).
Sampling them yields the K draft tokens d[b,k] and the drafter distribution
q[b,k,:] that the next verify uses in its acceptance test ("Project 14 -
speculative decoding inference server", section 架构: the draft model proposes
k tokens that the target then checks).

Readings (the pages give no formula for this step):

* D1  q = softmax(z / T_b) over the drafter's vocabulary, in fp64, at the
      request's temperature T_b -- the same reading as for the target side:
      the drafter samples at the request's temperature.
* D2  T_b = 0 selects greedy drafting: d is the lowest-index argmax and q is
      one-hot at d (the T -> 0 limit of D1 when the maximum is unique).
* D3  the draw is the inverse CDF of q in vocabulary order with one uniform
      per draft, strict comparison -- the sampler the verify's final draw uses.
* D4  row_index[b,k] names the drafter logit row of draft k of sequence b
      (the build's sample_rows); without it, draft k of sequence b is row
      b*K + k.
"""
from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np

from .verify import _draw_candidates, decode_logits, first_argmax, inverse_cdf, target_distribution


def draft_distribution(z_row: np.ndarray, T: float) -> np.ndarray:
    """q for one drafter row: softmax(z/T) for T > 0 (D1), one-hot at the
    lowest-index argmax for T = 0 (D2)."""
    z = np.asarray(z_row, dtype=np.float64)
    if T == 0.0:
        q = np.zeros(z.shape[0], dtype=np.float64)
        q[first_argmax(z)] = 1.0
        return q
    if not (T > 0.0 and np.isfinite(T)):
        raise ValueError(f"temperature must be 0 or finite and positive, got {T}")
    return target_distribution(z, T)


def draft_sample_row(z_row: np.ndarray, T: float, u: float) -> Tuple[int, np.ndarray]:
    """(d, q) for one drafter row: q by D1/D2, d drawn from q with u (D3)."""
    q = draft_distribution(z_row, T)
    if T == 0.0:
        return int(np.argmax(q)), q
    d, _, _ = inverse_cdf(q, float(u))
    return d, q


def _rows(B: int, K: int, row_index: Optional[np.ndarray]) -> np.ndarray:
    if row_index is None:
        return np.arange(B * K, dtype=np.int64).reshape(B, K)
    return np.asarray(row_index, dtype=np.int64).reshape(B, K)


def _temps(B: int, temperature: float, temperatures: Optional[np.ndarray]) -> np.ndarray:
    if temperatures is None:
        return np.full(B, np.float64(np.float32(temperature)))
    return np.asarray(temperatures, dtype=np.float32).astype(np.float64)


def draft_sample(logits: np.ndarray, dtype: str, uniforms: np.ndarray, temperature: float,
                 B: int, K: int, row_index: Optional[np.ndarray] = None,
                 temperatures: Optional[np.ndarray] = None):
    """Draft tokens [B, K] int32 and draft probabilities [B, K, V] fp64.

    logits: [R, V] drafter rows (fp32 values or bf16 bits), uniforms [B, K]
    fp32; temperatures, if given, [B] fp32 per sequence and override the
    scalar temperature (0 = greedy drafting for that sequence).
    """
    rows = _rows(B, K, row_index)
    Ts = _temps(B, temperature, temperatures)
    V = logits.shape[-1]
    d = np.empty((B, K), dtype=np.int32)
    q = np.empty((B, K, V), dtype=np.float64)
    for b in range(B):
        for k in range(K):
            z = decode_logits(logits[rows[b, k]], dtype)
            d[b, k], q[b, k] = draft_sample_row(z, Ts[b], uniforms[b, k])
    return d, q


def draft_outcomes(z_row: np.ndarray, T: float, u: float, tol: float = 1e-6) -> List[int]:
    """Draft tokens an evaluation exact up to ``tol`` may return for one row:
    those whose CDF cell lies within tol of u*S (D3); for T = 0 the argmax."""
    q = draft_distribution(z_row, T)
    if T == 0.0:
        return [int(np.argmax(q))]
    return _draw_candidates(q, float(u), tol)


def draft_probs(logits: np.ndarray, dtype: str, temperature: float, B: int, K: int,
                row_index: Optional[np.ndarray] = None,
                temperatures: Optional[np.ndarray] = None) -> np.ndarray:
    """q [B, K, V] fp64 of the drafter rows (D1, D2, D4), without drawing."""
    rows = _rows(B, K, row_index)
    Ts = _temps(B, temperature, temperatures)
    V = logits.shape[-1]
    q = np.empty((B, K, V), dtype=np.float64)
    for b in range(B):
        for k in range(K):
            q[b, k] = draft_distribution(decode_logits(logits[rows[b, k]], dtype), Ts[b])
    return q
