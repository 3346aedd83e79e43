"""Oracle checks of the high-concurrency batch (B=1024, K=7, V=151936 bf16),
run in worker processes for the full-size GPU parity tests.

Each task regenerates its sequences from their own seeded streams (synth draws
every sequence from a stream keyed by its index, so a subset regenerates
bit for bit) and returns what the oracle computes for them; the test process
compares the GPU outputs with the results.  Nothing here touches the GPU.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

TOL = 1e-6


def _inputs(lo: int, hi: int):
    return synth.make_verify_inputs(synth.verify_config(5), seqs=range(lo, hi), workers=1)


def _accept_flags(z64, q, d, u, T) -> int:
    """Accept tests of the canonical path that lie within TOL of their ratio."""
    tr = oracle.verify_sample_seq(z64, q, d, u, T)
    return sum(1 for k, r in enumerate(tr.ratios)
               if np.isfinite(r) and abs(np.float64(u[k]) - r) < TOL)


def verify_task(args):
    """(lo, hi, temps or None, gpu_tokens [n][K+1], gpu_acc [n], gpu_pd [n][K])
    -> list of error strings and (flags, accept_flags) totals.  temps None:
    uniform temperature (the sampled verify); else per-sequence temperatures
    (the mixed verify)."""
    lo, hi, temps, out, acc, pd = args
    vi = _inputs(lo, hi)
    K = vi.spec.K
    errors, flags, aflags = [], 0, 0
    for i in range(hi - lo):
        b = lo + i
        z64 = vi.logits_f64(i)
        q, d, u = vi.draft_probs[i], vi.draft_tokens[i], vi.uniforms[i]
        T = vi.temperature if temps is None else float(temps[i])
        if temps is not None and oracle.mixed.is_greedy(temps[i]):
            a, w_out, w_pd = oracle.mixed.verify_mixed_seq(z64, q, d, u, temps[i])
            if int(acc[i]) != a or not np.array_equal(out[i], w_out):
                errors.append(f"seq {b}: greedy ({int(acc[i])}, {out[i].tolist()}) != ({a}, {w_out.tolist()})")
            if not np.array_equal(pd[i], w_pd.astype(np.float32)):
                errors.append(f"seq {b}: greedy p_draft")
            continue
        canon, allowed, f = oracle.sample_outcomes(z64, q, d, u, T, tol=TOL)
        flags += f
        aflags += _accept_flags(z64, q, d, u, T)
        a = int(acc[i])
        if not 0 <= a <= K or (a, int(out[i, a])) not in allowed:
            errors.append(f"seq {b}: ({a}, {int(out[i, min(max(a, 0), K)])}) not in {allowed}")
            continue
        if not np.array_equal(out[i, :a], d[:a]) or not np.all(out[i, a + 1:] == -1):
            errors.append(f"seq {b}: malformed row {out[i].tolist()}")
        if (a, int(out[i, a])) != canon and f == 0:
            errors.append(f"seq {b}: departs from the canonical outcome without a near tie")
        want = np.array([oracle.target_distribution(z64[k], T)[int(d[k])] for k in range(K)])
        if not np.allclose(pd[i], want, rtol=1e-5, atol=1e-30):
            errors.append(f"seq {b}: p_draft {pd[i].tolist()} vs {want.tolist()}")
    return errors, flags, aflags


def greedy_task(args):
    """(lo, hi, gpu_tokens, gpu_acc) -> errors against oracle.verify_greedy."""
    lo, hi, out, acc = args
    vi = _inputs(lo, hi)
    w_out, w_acc = oracle.verify_greedy(vi.logits, "bf16", vi.draft_tokens)
    errors = [f"seq {lo + i}" for i in range(hi - lo)
              if int(acc[i]) != int(w_acc[i]) or not np.array_equal(out[i], w_out[i])]
    return errors


def draft_task(args):
    """(lo, hi, T, uniforms [n][K], gpu tokens [n][K], path of the GPU's q
    [B][K][V] fp32 (.npy, memory-mapped)) -> errors: every drafted row's q
    against the oracle's drafter distribution (1e-5 relative) and its token
    among the oracle's acceptable draws.  The drafter rows are the first K
    logit rows of each sequence."""
    lo, hi, T, u, tok, q_path = args
    vi = _inputs(lo, hi)
    K = vi.spec.K
    q_gpu = np.load(q_path, mmap_mode="r")
    errors = []
    for i in range(hi - lo):
        b = lo + i
        for k in range(K):
            z64 = oracle.decode_logits(vi.logits[i, k], "bf16")
            qo = oracle.draft.draft_distribution(z64, T)
            if not np.allclose(q_gpu[b, k], qo, rtol=1e-5, atol=1e-30):
                errors.append(f"seq {b} row {k}: q")
            if int(tok[i, k]) not in oracle.draft_outcomes(z64, T, float(u[i, k]), tol=TOL):
                errors.append(f"seq {b} row {k}: token {int(tok[i, k])}")
    return errors


def lq_task(args):
    """(lo, hi, T, drafter uniforms [n][K], gpu drafted tokens [n][K], gpu
    verify tokens, acc, pd) -> (errors, compared, flags): the decode round
    with q from the drafter logits, against the oracle's drafter and verify
    (sequences whose GPU draft differs from the oracle's, a near tie of the
    drafter's own draw, are skipped and counted)."""
    lo, hi, T, ud, tok, out, acc, pd = args
    vi = _inputs(lo, hi)
    K = vi.spec.K
    Td = float(np.float32(T))
    errors, compared, flags = [], 0, 0
    for i in range(hi - lo):
        b = lo + i
        drafted = [oracle.draft.draft_sample_row(oracle.decode_logits(vi.logits[i, k], "bf16"),
                                                 Td, ud[i, k]) for k in range(K)]
        od = np.array([x[0] for x in drafted], np.int32)
        if not np.array_equal(tok[i], od):
            continue
        oq = np.stack([x[1] for x in drafted])
        z64 = vi.logits_f64(i)
        canon, allowed, f = oracle.sample_outcomes(z64, oq, od, vi.uniforms[i], T, tol=TOL)
        flags += f
        a = int(acc[i])
        if not 0 <= a <= K or (a, int(out[i, a])) not in allowed:
            errors.append(f"seq {b}: ({a}, {int(out[i, min(max(a, 0), K)])}) not in {allowed}")
        want = np.array([oracle.target_distribution(z64[k], T)[int(od[k])] for k in range(K)])
        if not np.allclose(pd[i], want, rtol=1e-5, atol=1e-30):
            errors.append(f"seq {b}: p_draft")
        compared += 1
    return errors, compared, flags
