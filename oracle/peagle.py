"""Oracle: the P-EAGLE parallel-draft batch, one sequence and one row at a time.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

Source: the P-EAGLE / TorchSpec blog summary (blog.hotdry.top).
  * Section 并行架构的核心创新 (parallel architecture): the drafter's input
    pairs each prompt position's token embedding with that position's hidden
    state, pairs the newly generated token with h_context, and fills the
    multi-token-prediction positions 2..K with two shared learned
    placeholders, the MASK token embedding and h_shared; one forward over all
    positions predicts t1..tK.
  * Section TorchSpec 集成与工程优化 (engineering): inserting MASK
    placeholders makes the draft batch a different shape from the verify
    batch; its metadata (copy / scatter / insert / pad / mask / remap) is
    rebuilt on the GPU, a dedicated copy broadcasts h_shared into the mask
    slots, valid tokens keep normal KV slots and rejected tokens get
    PADDING_SLOT_ID = -1 so they write nothing to the KV cache.

Layout (a reading; the pages fix no row layout).  Each sequence owns a static
block of 2K rows (so the draft batch has a fixed shape, matching the CUDA-graph
range that the same section extends by K x max_num_seqs).  With a accepted
drafts, new token c, verify-slot-0 position L, and the EAGLE pairing "token
emitted after position p goes with the hidden state at p":

  rows 0..a-1        accepted    id d[r]        pos L+r        hidden h[r]        slot(L+r)
  row  a             NTP         id c           pos L+a        hidden h[a]        slot(L+a)
  rows a+m, m=1..K-1 MASK        id MASK        pos L+a+m      hidden h_shared    slot(L+a+m)
  rows a+K+j         rejected    id d[a+j]      pos L+a+1+j    hidden h[a+1+j]    -1
                     j=0..K-a-1

h[i] is the target hidden state of verify slot i (row b*(K+1)+i); slot(pos) =
block_table[b][pos // block_size] * block_size + pos % block_size (paged KV
cache, the serving default named in the rskf.cn survey, section 6).
sample_rows[b,k] = b*2K + a + k are the K rows (NTP and the K-1 MASK rows)
whose drafter outputs are t1..tK.

Parity of the row order itself is unpinned by the pages; the invariants in
the section descriptions above are what pins it.
"""
from __future__ import annotations

import numpy as np

PADDING_SLOT_ID = -1


def slot_of(block_row: np.ndarray, pos: int, block_size: int) -> int:
    """KV-cache slot of ``pos`` through one sequence's block table."""
    return int(block_row[pos // block_size]) * block_size + pos % block_size


def sequence_rows(a: int, K: int):
    """The 2K (role, r_token, pos_offset, hidden_slot) tuples of one sequence.

    role: "accepted" | "ntp" | "mask" | "rejected"; r_token indexes the draft
    (or -1 for the new token / MASK); pos_offset is added to L; hidden_slot is
    the verify slot whose hidden state is copied, or -1 for h_shared.
    """
    rows = []
    for r in range(a):
        rows.append(("accepted", r, r, r))
    rows.append(("ntp", -1, a, a))
    for m in range(1, K):
        rows.append(("mask", -1, a + m, -1))
    for j in range(K - a):
        rows.append(("rejected", a + j, a + 1 + j, a + 1 + j))
    assert len(rows) == 2 * K
    return rows


def build_draft_batch(out_tokens: np.ndarray, num_accepted: np.ndarray,
                      draft_tokens: np.ndarray, start_pos: np.ndarray,
                      block_table: np.ndarray, block_size: int,
                      target_hidden: np.ndarray, h_shared: np.ndarray,
                      mask_token_id: int):
    """Build the P-EAGLE drafter batch for B sequences.

    Hidden states are treated as raw element bits (any dtype): the step is a
    copy, so equality is bitwise.  Returns a dict with input_ids [B*2K] int32,
    positions [B*2K] int64, slot_mapping [B*2K] int64, hidden [B*2K, H],
    sample_rows [B, K] int32, hidden_src [B*2K] int64 (-1 = h_shared).
    """
    B, K = draft_tokens.shape
    H = target_hidden.shape[1]
    n = B * 2 * K
    ids = np.empty(n, dtype=np.int32)
    pos = np.empty(n, dtype=np.int64)
    slots = np.empty(n, dtype=np.int64)
    src = np.empty(n, dtype=np.int64)
    hid = np.empty((n, H), dtype=target_hidden.dtype)
    sample_rows = np.empty((B, K), dtype=np.int32)
    for b in range(B):
        a = int(num_accepted[b])
        assert 0 <= a <= K
        L = int(start_pos[b])
        c = int(out_tokens[b, a])
        base = b * 2 * K
        for i, (role, rt, po, hs) in enumerate(sequence_rows(a, K)):
            row = base + i
            if role == "accepted":
                ids[row] = int(out_tokens[b, rt])
            elif role == "ntp":
                ids[row] = c
            elif role == "mask":
                ids[row] = mask_token_id
            else:
                ids[row] = int(draft_tokens[b, rt])
            pos[row] = L + po
            slots[row] = (PADDING_SLOT_ID if role == "rejected"
                          else slot_of(block_table[b], L + po, block_size))
            if hs < 0:
                src[row] = -1
                hid[row] = h_shared
            else:
                src[row] = b * (K + 1) + hs
                hid[row] = target_hidden[b * (K + 1) + hs]
        for k in range(K):
            sample_rows[b, k] = base + a + k
    return {"input_ids": ids, "positions": pos, "slot_mapping": slots,
            "hidden": hid, "sample_rows": sample_rows, "hidden_src": src}
