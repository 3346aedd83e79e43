"""Pins for the oracle's P-EAGLE draft batch.

What the P-EAGLE summary (blog.hotdry.top) fixes, checked on random batches:
 (i)   positions 2..K of the multi-token prediction use the MASK token and
       h_shared: exactly K-1 MASK rows per sequence, each carrying h_shared
       (section 并行架构的核心创新);
 (ii)  the new token is paired with h_context, the hidden state of the slot
       that produced it (same section);
 (iii) valid tokens get normal KV slots and rejected tokens PADDING_SLOT_ID =
       -1 (section TorchSpec 集成与工程优化): exactly K-a_b rows with -1 per
       sequence, and every other slot is a real slot;
 (iv)  the rows that write KV (valid + MASK) sit at distinct, contiguous
       positions from L_b, and their slots are pairwise distinct across the
       batch (distinct positions map to distinct paged-KV slots);
 (v)   every hidden row is bitwise one of the target hidden rows of its own
       sequence or h_shared; a = K leaves no -1 and a = 0 leaves K of them;
 (vi)  each prompt-side position pairs its token with the hidden state of the
       corresponding position (section 并行架构的核心创新): read with the EAGLE
       shift, the valid rows in position order carry the emitted tokens
       out[0..a] and the hidden rows h[0..a].
The slot formula is checked by brute force against a dense position -> slot
map built from the block table.
"""
import numpy as np
import pytest

from oracle import PADDING_SLOT_ID, build_draft_batch


def _case(rng, B, K, H, bs, V=1000, a=None):
    L = rng.integers(1, 300, size=B).astype(np.int64)
    nblk = (L + 2 * K + bs - 1) // bs
    pool = rng.permutation(int(nblk.sum()) + 7).astype(np.int32)
    bt = np.full((B, int(nblk.max()) + 2), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :nblk[b]] = pool[off:off + nblk[b]]
        off += int(nblk[b])
    acc = rng.integers(0, K + 1, size=B).astype(np.int32) if a is None else np.full(B, a, np.int32)
    d = rng.integers(0, V, size=(B, K)).astype(np.int32)
    out = np.full((B, K + 1), -1, dtype=np.int32)
    for b in range(B):
        out[b, :acc[b]] = d[b, :acc[b]]
        out[b, acc[b]] = rng.integers(0, V)
    hid = rng.integers(0, 2 ** 16, size=(B * (K + 1), H)).astype(np.uint16)
    hs = rng.integers(0, 2 ** 16, size=H).astype(np.uint16)
    return dict(out_tokens=out, num_accepted=acc, draft_tokens=d, start_pos=L,
                block_table=bt, block_size=bs, target_hidden=hid, h_shared=hs,
                mask_token_id=V + 5)


def check_invariants(res, case, K):
    B = case["draft_tokens"].shape[0]
    ids, pos, slots, hid = res["input_ids"], res["positions"], res["slot_mapping"], res["hidden"]
    assert ids.shape == (B * 2 * K,)
    mask_id = case["mask_token_id"]
    all_valid_slots = []
    for b in range(B):
        a = int(case["num_accepted"][b])
        L = int(case["start_pos"][b])
        seg = slice(b * 2 * K, (b + 1) * 2 * K)
        sid, spos, sslot, shid = ids[seg], pos[seg], slots[seg], hid[seg]
        is_mask = sid == mask_id
        assert is_mask.sum() == K - 1                                     # (i)
        assert np.all(shid[is_mask] == case["h_shared"])                  # (i)
        is_pad = sslot == PADDING_SLOT_ID
        assert is_pad.sum() == K - a                                      # (iii)
        writes = ~is_pad
        assert np.array_equal(np.sort(spos[writes]), L + np.arange(a + K))   # (iv)
        all_valid_slots.extend(sslot[writes].tolist())
        # (ii): the row carrying the new token c holds h[a] of this sequence
        c = int(case["out_tokens"][b, a])
        hrows = case["target_hidden"][b * (K + 1):(b + 1) * (K + 1)]
        ntp = [i for i in range(2 * K) if sid[i] == c and spos[i] == L + a and not is_pad[i]]
        assert ntp and any(np.array_equal(shid[i], hrows[a]) for i in ntp)
        # (vi): the valid rows (neither MASK nor padding), in position order,
        # pair the emitted tokens out[0..a] with the hidden rows h[0..a]
        valid = np.nonzero(writes & ~is_mask)[0]
        valid = valid[np.argsort(spos[valid], kind="stable")]
        assert np.array_equal(sid[valid], case["out_tokens"][b, :a + 1])
        assert np.array_equal(shid[valid], hrows[:a + 1])
        # (v): every hidden row is one of this sequence's or h_shared
        for i in range(2 * K):
            assert is_mask[i] or any(np.array_equal(shid[i], h) for h in hrows)
        # sample rows: K distinct rows, the NTP row first, then the MASK rows
        sr = res["sample_rows"][b] - b * 2 * K
        assert len(set(sr.tolist())) == K
        assert sid[sr[0]] == c and np.all(sid[sr[1:]] == mask_id)
        # rejected drafts keep their own tokens
        assert sorted(sid[is_pad].tolist()) == sorted(case["draft_tokens"][b, a:].tolist())
    assert len(set(all_valid_slots)) == len(all_valid_slots)              # (iv)


@pytest.mark.parametrize("B,K,H,bs,seed", [(1, 1, 4, 16, 0), (5, 3, 8, 4, 1), (40, 7, 16, 16, 2),
                                           (9, 7, 3, 1, 3)])
def test_invariants_random(B, K, H, bs, seed):
    rng = np.random.default_rng(seed)
    case = _case(rng, B, K, H, bs)
    check_invariants(build_draft_batch(**case), case, K)


@pytest.mark.parametrize("a", [0, 7])
def test_extreme_accept_counts(a):
    rng = np.random.default_rng(10 + a)
    K = 7
    case = _case(rng, 6, K, 8, 16, a=a)
    res = build_draft_batch(**case)
    check_invariants(res, case, K)
    n_pad = int((res["slot_mapping"] == PADDING_SLOT_ID).sum())
    assert n_pad == (0 if a == K else 6 * K)


def check_slots_dense(res, case, K):
    """Every real slot equals the dense position -> slot map of the sequence's pages."""
    bs = case["block_size"]
    B = case["draft_tokens"].shape[0]
    for b in range(B):
        # dense map: position p of sequence b lives in page table[p // bs] at offset p % bs
        dense = {}
        for blk_i, blk in enumerate(case["block_table"][b]):
            if blk < 0:
                continue
            for o in range(bs):
                dense[blk_i * bs + o] = int(blk) * bs + o
        for i in range(2 * K):
            row = b * 2 * K + i
            s = int(res["slot_mapping"][row])
            if s != PADDING_SLOT_ID:
                assert s == dense[int(res["positions"][row])]


def test_slot_formula_brute_force():
    rng = np.random.default_rng(12)
    K = 5
    case = _case(rng, 12, K, 2, 8)
    check_slots_dense(build_draft_batch(**case), case, K)


def test_worked_example():
    # One sequence, K = 3, two drafts (11, 12, 13) of which the first is
    # accepted, new token 42, verify slot 0 at position 10, 4-token pages.
    K, bs = 3, 4
    hid = np.arange(4 * 2, dtype=np.uint16).reshape(4, 2) + 100   # h[i] = (100+2i, 101+2i)
    case = dict(out_tokens=np.array([[11, 42, -1, -1]], np.int32),
                num_accepted=np.array([1], np.int32),
                draft_tokens=np.array([[11, 12, 13]], np.int32),
                start_pos=np.array([10], np.int64),
                block_table=np.array([[7, 2, 9, 5]], np.int32), block_size=bs,
                target_hidden=hid, h_shared=np.array([1, 2], np.uint16), mask_token_id=99)
    res = build_draft_batch(**case)
    # accepted draft 11 with h[0] at position 10 (page 9, offset 2 -> slot 38);
    # new token 42 with h_context = h[1] at 11 (slot 39); two MASK rows with
    # h_shared at 12, 13 (page 5 -> slots 20, 21); rejected drafts 12, 13
    # with their own hidden rows h[2], h[3] at 12, 13 and slot -1.
    assert res["input_ids"].tolist() == [11, 42, 99, 99, 12, 13]
    assert res["positions"].tolist() == [10, 11, 12, 13, 12, 13]
    assert res["slot_mapping"].tolist() == [38, 39, 20, 21, -1, -1]
    assert res["hidden"].tolist() == [[100, 101], [102, 103], [1, 2], [1, 2], [104, 105], [106, 107]]
    assert res["sample_rows"].tolist() == [[1, 2, 3]]
