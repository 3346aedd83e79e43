"""CPU oracle for speculative verify-and-accept and the P-EAGLE draft batch.

TEST INFRASTRUCTURE ONLY.  Plain, slow, fp64 numpy, one sequence at a time.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it; the product path (``draft_verification_vocab_amd``
and its HIP library) never does, and this package imports nothing from it.

What each function follows (the pages cited are the three source pages:
"Project 14 - speculative decoding inference server" (ai-engineering.com.cn),
the P-EAGLE / TorchSpec blog summary (blog.hotdry.top), and the rskf.cn survey
of Eagle / MTP / DFlash / DSPark):

* ``verify.target_distribution``  softmax of a logit row at temperature T.
  Pinned by closed forms and scipy (tests/test_oracle_softmax.py).
* ``verify.verify_greedy``        argmax-match prefix, then the target argmax.
  Pinned by the argmax-chain property and brute force.
* ``verify.verify_sample``        p/q acceptance, first-rejection prefix,
  residual max(0, p - q) resample or bonus draw from p.  Pinned by exact
  enumeration of the output law on tiny vocabularies, chi-square and binomial
  tests, closed forms for the acceptance rate and mean accepted length, and
  special cases (q = p, q one-hot on a zero of p, disjoint supports).
* ``draft.draft_sample``          the drafter's K prediction rows per sequence
  -> draft tokens and draft probabilities q for the next verify (softmax at
  the request's temperature, inverse-CDF draw; T = 0 drafts greedily).
  Pinned by scipy's softmax, numpy's searchsorted, cell-midpoint brute force,
  chi-square, and by the end-to-end law: drafting with it and verifying with
  ``verify_sample`` emits tokens distributed as the target.
* ``mixed.verify_mixed``          a verify batch with a temperature per
  sequence (0 = greedy).  Pinned by per-group chi-square against scipy's
  softmax at each group's temperature, the exact greedy argmax chain inside a
  mixed batch, the fp32 boundary of invalid temperatures, and reduction to
  ``verify_sample`` / ``verify_greedy`` for uniform batches.
* ``metrics.counters`` / ``rates``  acceptance counters of verify calls and the
  acceptance length, tokens per round, draft acceptance rate and conditional
  per-position rates.  Pinned by a hand-counted example, the closed forms of
  independent acceptance (truncated geometric), and the verify oracle's
  all-accept / all-reject cases.
* ``tree.verify_tree_*``          verification of a draft tree (greedy argmax
  walk; recursive rejection over independently drafted children).  Pinned
  by reduction to the chain verify when every node has one child, the exact
  law of the first emitted token on star trees (bisection over the uniforms,
  equal to the target softmax), chi-square on two-level trees, and a brute
  force check of the greedy walk.
* ``peagle.build_draft_batch``    the P-EAGLE drafter batch.  Pinned by the
  invariants the P-EAGLE summary fixes (K-1 MASK rows per sequence, slot -1
  exactly on rejected tokens, h_shared on the MASK rows, the new token paired
  with h_context) and by brute-force checks of the slot formula.  The row
  order inside a sequence (accepted, NTP, MASK, rejected) and the content of
  the rejected padding rows are readings the pages leave open: those two
  aspects are parity unpinned by the pages.
"""
from . import draft, metrics, mixed, peagle, tree, verify  # noqa: F401
from .mixed import verify_mixed  # noqa: F401
from .draft import draft_distribution, draft_outcomes, draft_sample  # noqa: F401
from .peagle import PADDING_SLOT_ID, build_draft_batch  # noqa: F401
from .verify import (  # noqa: F401
    decode_logits,
    first_argmax,
    sample_outcomes,
    target_distribution,
    verify_greedy,
    verify_sample,
    verify_sample_seq,
)
