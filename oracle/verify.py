"""Oracle: batched speculative verify-and-accept, fp64, one sequence at a time.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

Notation.  A batch holds B sequences with K draft tokens each.  Target logits
are [B, K+1, V]; row k of sequence b is the target's distribution for the
token that follows verify slot k, so draft d[b,k] is tested against row k and
row K yields the bonus token when every draft is accepted.  Draft
probabilities q are [B, K, V] and are used as given.  Uniforms are [B, K+1]:
u[b,k] (k < K) decides draft k, u[b,K] drives the single final draw.

The flow is the verify pass of "Project 14 - speculative decoding inference
server" (section 架构, architecture): the target checks all k drafts in one
forward, the accepted prefix is kept and the rejected suffix is resampled.
Section 概念 (concepts) of the same page fixes that an accepted prefix replaces
the greedy path.  The rskf.cn survey (sections 1 and 2.2) states the property
that makes the method lossless: the output equals plain autoregressive
decoding of the target.  The pages give no formulas; the steps below are the
plainest reading consistent with that property, each reading named where it
is taken.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np


# ---------------------------------------------------------------- inputs
def decode_logits(z: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored logits to fp64 exactly.

    ``dtype`` is "f32" (float32 values) or "bf16" (uint16 bit patterns: the
    top half of an IEEE binary32, so shifting them left by 16 bits is exact).
    """
    if dtype == "f32":
        return np.asarray(z, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        bits = np.asarray(z, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(f"unknown logits dtype {dtype!r}")


# ---------------------------------------------------------------- target side
def target_distribution(z_row: np.ndarray, T: float) -> np.ndarray:
    """p(v) = exp((z_v - m)/T) / sum_w exp((z_w - m)/T), m = max z, in fp64.

    The decode-time softmax over the vocabulary named in the rskf.cn survey,
    section 2.1 (temperature sampling over the vocab).  T is the request's
    temperature widened to fp64; the drafter's probabilities are not rescaled.
    """
    z = np.asarray(z_row, dtype=np.float64)
    m = z.max()
    e = np.exp((z - m) / np.float64(T))
    return e / e.sum()


def first_argmax(z_row: np.ndarray) -> int:
    """Lowest index attaining the row maximum (numpy's argmax keeps the first).

    Reading: the pages fix no tie rule; the lowest index is the plainest
    deterministic one.
    """
    return int(np.argmax(np.asarray(z_row, dtype=np.float64)))


# ---------------------------------------------------------------- greedy
def verify_greedy_seq(z_rows: np.ndarray, d: Sequence[int]) -> Tuple[int, int]:
    """Greedy verify of one sequence: (a, c).

    a is the first k < K whose draft differs from the target argmax g_k of row
    k (K when every draft matches); c = g_a is the target's own token after
    the accepted prefix (Project 14, section 概念: the accepted prefix replaces
    the greedy path, so the emitted tokens are exactly the target's greedy
    continuation).  Temperature plays no part.
    """
    K = len(d)
    for k in range(K):
        g = first_argmax(z_rows[k])
        if int(d[k]) != g:
            return k, g
    return K, first_argmax(z_rows[K])


def assemble(d: Sequence[int], a: int, c: int) -> np.ndarray:
    """out_tokens row: accepted drafts d[0..a-1], the new token c, then -1.

    Reading: -1 marks the unused tail, mirroring PADDING_SLOT_ID = -1 of the
    P-EAGLE summary (section TorchSpec 集成与工程优化).
    """
    K = len(d)
    out = np.full(K + 1, -1, dtype=np.int32)
    out[:a] = np.asarray(d[:a], dtype=np.int32)
    out[a] = c
    return out


def verify_greedy(logits: np.ndarray, dtype: str, draft_tokens: np.ndarray):
    """Batch greedy verify.  Returns (out_tokens [B,K+1] int32, num_accepted [B] int32)."""
    B, K1, V = logits.shape
    K = K1 - 1
    out = np.empty((B, K + 1), dtype=np.int32)
    acc = np.empty(B, dtype=np.int32)
    for b in range(B):
        z = decode_logits(logits[b], dtype)
        d = draft_tokens[b]
        assert all(0 <= int(x) < V for x in d), "draft token outside the vocabulary"
        a, c = verify_greedy_seq(z, d)
        out[b] = assemble(d, a, c)
        acc[b] = a
    return out, acc


# ---------------------------------------------------------------- sampling
def accept_ratio(p_x: float, q_x: float) -> float:
    """p(x)/q(x); with q(x) = 0 the ratio is +inf when p(x) > 0 and 0 otherwise.

    Reading: a draft the drafter gave zero probability (after fp32 rounding)
    is kept when the target allows it and rejected when it does not.
    """
    if q_x > 0.0:
        return p_x / q_x
    return np.inf if p_x > 0.0 else 0.0


def residual(p: np.ndarray, q: np.ndarray) -> np.ndarray:
    """Unnormalised resampling mass r(v) = max(0, p(v) - q(v)) (Project 14,
    section 架构: the rejected suffix is resampled; the residual is the part
    of p that the accepted draws did not already cover)."""
    return np.maximum(0.0, p - q)


def inverse_cdf(r: np.ndarray, u: float) -> Tuple[int, float, np.ndarray]:
    """Draw from the unnormalised mass r with one uniform u in [0, 1).

    S is the running total of r in vocabulary order; the draw is the smallest
    v whose running total exceeds u*S.  The comparison is strict, so a token
    with zero mass is never returned; if rounding leaves no such v, the
    largest v with positive mass is returned.  Reading: the pages fix no
    sampler; inverse-CDF over vocabulary order is the plainest exact one.
    Returns (v, S, cdf).
    """
    cdf = np.cumsum(np.asarray(r, dtype=np.float64))
    S = float(cdf[-1])
    target = np.float64(u) * S
    hit = np.nonzero(cdf > target)[0]
    if hit.size:
        return int(hit[0]), S, cdf
    pos = np.nonzero(r > 0.0)[0]
    return int(pos[-1]), S, cdf


@dataclasses.dataclass
class SampleTrace:
    """Everything one sampled verify computes for a sequence."""
    a: int
    c: int
    out_tokens: np.ndarray
    p_draft: np.ndarray        # [K] p_k(d_k), for every k (not only the tested ones)
    ratios: List[float]        # ratios of the rows actually tested (0..min(a, K-1))
    draw_row: int              # row whose mass the final draw used
    draw_from_p: bool          # True: bonus (a = K) or degenerate residual -> p
    mass: np.ndarray           # the mass r the final draw used
    target: float              # u[K] * S
    cdf: np.ndarray


def verify_sample_seq(z_rows: np.ndarray, q_rows: np.ndarray, d: Sequence[int],
                      u: Sequence[float], T: float,
                      force: Optional[dict] = None) -> SampleTrace:
    """Sampled verify of one sequence.

    1. p_k = target_distribution(z_k, T) for k = 0..K.
    2. Walk k = 0..K-1: accept draft x = d_k iff u_k < p_k(x)/q_k(x) (strict;
       reading: with u in [0,1) a draft whose ratio is >= 1 is always kept).
       The first rejection fixes a = k; a = K when none is rejected.
    3. a < K: draw c from r = max(0, p_a - q_a); if that mass sums to 0 (only
       possible when q_a does not sum to 1) draw from p_a instead.
       a = K: draw the bonus token c from p_K.
       The draw uses the last uniform u_K (reading: one uniform per test, one
       for the final draw; tests after the first rejection are unused).
    ``force`` (test use) maps k -> bool to override a decision at row k.
    """
    K = len(d)
    V = z_rows.shape[1]
    p = [target_distribution(z_rows[k], T) for k in range(K + 1)]
    q = np.asarray(q_rows, dtype=np.float64)
    p_draft = np.array([p[k][int(d[k])] for k in range(K)], dtype=np.float64)
    ratios: List[float] = []
    a = K
    for k in range(K):
        x = int(d[k])
        assert 0 <= x < V, "draft token outside the vocabulary"
        ratio = accept_ratio(p[k][x], q[k, x])
        ratios.append(ratio)
        ok = np.float64(u[k]) < ratio
        if force is not None and k in force:
            ok = bool(force[k])
        if not ok:
            a = k
            break
    if a < K:
        mass = residual(p[a], q[a])
        from_p = not (mass.sum() > 0.0)
        if from_p:
            mass = p[a]
    else:
        mass, from_p = p[K], True
    c, S, cdf = inverse_cdf(mass, float(u[K]))
    return SampleTrace(a, c, assemble(d, a, c), p_draft, ratios, a, from_p, mass,
                       float(np.float64(u[K]) * S), cdf)


def verify_sample(logits: np.ndarray, dtype: str, draft_probs: np.ndarray,
                  draft_tokens: np.ndarray, uniforms: np.ndarray, T: float):
    """Batch sampled verify.

    Returns (out_tokens [B,K+1] int32, num_accepted [B] int32, p_draft [B,K] fp64).
    """
    B, K1, V = logits.shape
    K = K1 - 1
    assert T > 0.0
    out = np.empty((B, K + 1), dtype=np.int32)
    acc = np.empty(B, dtype=np.int32)
    pd = np.empty((B, K), dtype=np.float64)
    for b in range(B):
        tr = verify_sample_seq(decode_logits(logits[b], dtype), draft_probs[b],
                               draft_tokens[b], uniforms[b], T)
        out[b], acc[b], pd[b] = tr.out_tokens, tr.a, tr.p_draft
    return out, acc, pd


# ---------------------------------------------------------------- near ties
def _draw_candidates(mass: np.ndarray, u: float, tol: float) -> List[int]:
    """Tokens an exact-up-to-``tol`` evaluation of the final draw may return:
    those with positive mass whose CDF cell [cdf[v-1], cdf[v]) lies within tol
    of u*S.  With tol = 0 this is exactly the inverse_cdf result."""
    c0, S, cdf = inverse_cdf(mass, u)
    if tol <= 0.0:
        return [c0]
    target = np.float64(u) * S
    lo = np.concatenate([[0.0], cdf[:-1]])
    ok = (mass > 0.0) & (lo - tol <= target) & (target < cdf + tol)
    cand = set(int(v) for v in np.nonzero(ok)[0])
    cand.add(c0)
    return sorted(cand)


def sample_outcomes(z_rows: np.ndarray, q_rows: np.ndarray, d: Sequence[int],
                    u: Sequence[float], T: float, tol: float = 1e-6):
    """All (a, c) outcomes a correct evaluation may reach when every decision
    within ``tol`` of its threshold may go either way.

    An accept test is a near tie when |u_k - p_k(x)/q_k(x)| < tol; a final
    draw is a near tie when u*S lies within tol of a CDF boundary.  Returns
    (canonical (a, c), sorted list of acceptable (a, c), number of near ties).
    """
    K = len(d)
    p = [target_distribution(z_rows[k], T) for k in range(K + 1)]
    q = np.asarray(q_rows, dtype=np.float64)
    outcomes = set()
    flags = 0

    def final(a: int):
        nonlocal flags
        if a < K:
            mass = residual(p[a], q[a])
            if not (mass.sum() > 0.0):
                mass = p[a]
        else:
            mass = p[K]
        cands = _draw_candidates(mass, float(u[K]), tol)
        if len(cands) > 1:
            flags += 1
        for c in cands:
            outcomes.add((a, c))

    def walk(k: int):
        nonlocal flags
        if k == K:
            final(K)
            return
        ratio = accept_ratio(p[k][int(d[k])], q[k, int(d[k])])
        uk = np.float64(u[k])
        near = np.isfinite(ratio) and abs(uk - ratio) < tol
        if near:
            flags += 1
            walk(k + 1)
            final(k)
        elif uk < ratio:
            walk(k + 1)
        else:
            final(k)

    walk(0)
    tr = verify_sample_seq(z_rows, q_rows, d, u, T)
    canonical = (tr.a, tr.c)
    assert canonical in outcomes
    return canonical, sorted(outcomes), flags
