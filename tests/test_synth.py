"""Seeded generators: determinism, subset regeneration, and the acceptance
ranges the workloads are meant to have."""
import numpy as np
import pytest

import synth
from oracle import target_distribution


def test_same_seed_same_bytes():
    a = synth.make_verify_inputs(synth.verify_config(2))
    b = synth.make_verify_inputs(synth.verify_config(2))
    for x, y in [(a.logits, b.logits), (a.draft_probs, b.draft_probs),
                 (a.draft_tokens, b.draft_tokens), (a.uniforms, b.uniforms)]:
        assert x.tobytes() == y.tobytes()


def test_subset_regenerates_identically():
    spec = synth.verify_config(2)
    full = synth.make_verify_inputs(spec)
    sub = synth.make_verify_inputs(spec, seqs=[6, 1])
    assert np.array_equal(sub.logits[0], full.logits[6])
    assert np.array_equal(sub.draft_probs[1], full.draft_probs[1])
    assert np.array_equal(sub.draft_tokens[0], full.draft_tokens[6])


def test_workers_do_not_change_values():
    spec = synth.verify_config(2)
    one = synth.make_verify_inputs(spec, workers=1)
    two = synth.make_verify_inputs(spec, workers=2)
    assert one.logits.tobytes() == two.logits.tobytes()
    assert one.draft_tokens.tobytes() == two.draft_tokens.tobytes()


def test_bf16_rounding():
    x = np.array([1.0, 1.00390625, 1.01171875, -3.0e38, 1e-40], dtype=np.float32)
    bits = synth.f32_to_bf16_bits(x)
    # 1 + 2^-8 is halfway between 1 and 1 + 2^-7: ties to even -> 1.0
    assert bits[0] == 0x3F80 and bits[1] == 0x3F80
    assert bits[2] == 0x3F82          # 1 + 3*2^-8 -> 1 + 2^-6 (even)
    assert np.all(np.isfinite(synth.bf16_bits_to_f32(bits)))


def _mean_beta(vi, T, nseq):
    betas = []
    for i in range(nseq):
        z = vi.logits_f64(i)
        for k in range(vi.spec.K):
            p = target_distribution(z[k], T)
            betas.append(np.minimum(p, vi.draft_probs[i, k].astype(np.float64)).sum())
    return float(np.mean(betas))


def test_verify_mid_acceptance_range():
    vi = synth.make_verify_inputs(synth.verify_config(2))
    beta = _mean_beta(vi, 1.0, vi.spec.B)
    assert 0.60 <= beta <= 0.75                  # the ~60-75% the workload asks for


def test_large_vocab_sample_rows():
    spec = synth.verify_config(4)
    vi = synth.make_verify_inputs(spec, seqs=[0, 33])
    assert vi.logits.dtype == np.uint16 and vi.logits.shape == (2, 8, 201088)
    beta = _mean_beta(vi, spec.temperature, 2)
    assert 0.35 <= beta <= 0.75
    # drafts lie in the vocabulary and are likely under their own q
    assert np.all((vi.draft_tokens >= 0) & (vi.draft_tokens < spec.V))


def test_build_inputs_shapes():
    bi = synth.make_build_inputs(synth.build_config(3))
    s = bi.spec
    assert bi.target_hidden.shape == (s.B * (s.K + 1), s.H)
    assert bi.mask_token_id >= s.V
    assert np.all((bi.start_pos >= s.L_min) & (bi.start_pos <= s.L_max))
    need = (bi.start_pos + 2 * s.K + s.block_size - 1) // s.block_size
    for b in range(s.B):
        row = bi.block_table[b]
        assert np.all(row[:need[b]] >= 0) and np.all(row[need[b]:] == -1)
    used = bi.block_table[bi.block_table >= 0]
    assert len(np.unique(used)) == used.size
    for b in range(s.B):
        a = bi.num_accepted[b]
        assert np.array_equal(bi.out_tokens[b, :a], bi.draft_tokens[b, :a])
        assert np.all(bi.out_tokens[b, a + 1:] == -1)


def test_draft_inputs_shapes_and_determinism():
    from synth.workloads import DRAFT_CONFIGS, make_draft_inputs
    spec = DRAFT_CONFIGS["draft-ragged"]
    a = make_draft_inputs(spec)
    b = make_draft_inputs(spec)
    B, K, V, R = spec.B, spec.K, spec.V, spec.rows_per_seq
    assert a.logits.shape == (B * R, V) and a.logits.dtype == np.uint16
    assert np.array_equal(a.logits, b.logits) and np.array_equal(a.uniforms, b.uniforms)
    assert a.uniforms.shape == (B, K) and a.uniforms.dtype == np.float32
    assert ((a.uniforms >= 0) & (a.uniforms < 1)).all()
    # K distinct rows per sequence, all inside that sequence's block of rows
    for s in range(B):
        r = a.row_index[s]
        assert len(set(r.tolist())) == K
        assert ((r >= s * R) & (r < (s + 1) * R)).all()
    assert set(a.temperatures.tolist()) <= set(np.float32([0.0, 0.5, 0.7, 1.0, 1.3]).tolist())
    assert a.temperatures.dtype == np.float32
    t = make_draft_inputs(DRAFT_CONFIGS["draft-tiny"])
    assert t.row_index is None and t.temperatures is None and t.logits.dtype == np.float32


def test_mixed_temperatures():
    from synth import MIXED_TEMPERATURES, make_temperatures
    t = make_temperatures(200, 9)
    assert t.dtype == np.float32 and t.shape == (200,)
    assert set(t.tolist()) == set(np.float32(MIXED_TEMPERATURES).tolist())
    assert np.array_equal(t[:50], make_temperatures(50, 9))


def test_tree_inputs():
    from synth import TREE_CONFIGS, make_tree_inputs, static_tree_parents
    assert static_tree_parents((3, 2, 1)).tolist() == [0, 0, 0, 1, 1, 2, 2, 3, 3,
                                                       4, 5, 6, 7, 8, 9]
    for name in ("tree-tiny", "tree-mid"):
        ti = make_tree_inputs(TREE_CONFIGS[name])
        s = ti.spec
        assert ti.logits.shape == (s.B, s.N + 1, s.V) and ti.uniforms.shape == (s.B, s.N + 1)
        for b in range(s.B):
            assert all(0 <= ti.parents[b, i] <= i for i in range(s.N))   # parent of node i+1
        assert ((ti.tokens >= 0) & (ti.tokens < s.V)).all()
        assert np.allclose(ti.draft_probs.sum(axis=2), 1.0, atol=1e-5)
        again = make_tree_inputs(s)
        assert np.array_equal(again.tokens, ti.tokens) and np.array_equal(again.logits, ti.logits)


def test_tree_workers_do_not_change_values():
    from synth import TREE_CONFIGS, make_tree_inputs
    s = TREE_CONFIGS["tree-tiny"]
    a, b = make_tree_inputs(s, workers=1), make_tree_inputs(s, workers=2)
    for f in ("logits", "draft_probs", "parents", "tokens", "uniforms"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
