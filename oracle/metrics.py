"""Oracle: acceptance metrics of speculative decoding, counted from the accept
counts that verify returns.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

The pages name the quantities a deployment watches: the acceptance length,
the mean number of drafts the verifier accepts per speculation round (P-EAGLE
/ TorchSpec blog summary, section 监控与调优建议), and the acceptance rate and
accepted tokens per step of the decode log ("Project 14 - speculative
decoding inference server", section 使用它; Prometheus metrics in section
架构).

Readings: a round is one sequence in one verify call; it proposes K drafts,
accepts a of them and emits a + 1 tokens (the accepted drafts and the new
token).  The counters are integers, so they can be summed across calls; the
rates follow from them:
  acceptance length      = accepted / rounds
  tokens per round       = emitted / rounds
  draft acceptance rate  = accepted / proposed
  conditional rate at k  = #(a > k) / #(a >= k)   (draft k accepted, given
                            that it was tested)
The accept-count histogram holds every one of these.
"""
from __future__ import annotations

from typing import Dict, Sequence

import numpy as np


def counters(num_accepted: Sequence[int], K: int) -> Dict[str, object]:
    """Counters of one verify call: rounds, proposed, accepted, emitted and
    the histogram of accept counts (K+1 bins)."""
    a = np.asarray(num_accepted, dtype=np.int64)
    assert np.all((a >= 0) & (a <= K)), "accept count outside [0, K]"
    hist = np.zeros(K + 1, dtype=np.int64)
    for x in a:
        hist[x] += 1
    return {"steps": 1, "rounds": int(a.size), "proposed": int(a.size) * K,
            "accepted": int(a.sum()), "emitted": int(a.sum()) + int(a.size), "hist": hist}


def accumulate(total: Dict[str, object], step: Dict[str, object]) -> Dict[str, object]:
    """Counters summed over calls."""
    return {k: total[k] + step[k] for k in ("steps", "rounds", "proposed", "accepted",
                                            "emitted", "hist")}


def rates(c: Dict[str, object]) -> Dict[str, object]:
    """The derived quantities of the module docstring."""
    hist = np.asarray(c["hist"], dtype=np.int64)
    K = hist.size - 1
    reached = np.array([hist[k:].sum() for k in range(K)], dtype=np.float64)   # a >= k
    passed = np.array([hist[k + 1:].sum() for k in range(K)], dtype=np.float64)  # a > k
    with np.errstate(invalid="ignore", divide="ignore"):
        cond = np.where(reached > 0, passed / np.maximum(reached, 1), np.nan)
    R = c["rounds"]
    return {"acceptance_length": c["accepted"] / R if R else float("nan"),
            "tokens_per_round": c["emitted"] / R if R else float("nan"),
            "draft_acceptance_rate": c["accepted"] / c["proposed"] if c["proposed"] else float("nan"),
            "conditional_rate": cond}
