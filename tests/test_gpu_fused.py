"""GPU parity at full size: the fused high-concurrency step.

B=1024 sequences, K=7, V=151936 bf16 logits (2.49 GB) with fp32 draft
probabilities (4.36 GB), verified on the device, then the P-EAGLE batch (H=2048
bf16, prompt lengths U{64..8192}) built from the verify outputs on the same
stream with no host round trip.  Every sequence is checked for well-formed
output and the build invariants; a seeded sample of sequences is checked
against the oracle one by one (the oracle's cost limits the sample).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import DEV, check_sample_sequence, dev, host_bits
from tests.test_oracle_build import check_invariants

pytestmark = pytest.mark.gpu

N_SAMPLED = 12


@pytest.fixture(scope="module")
def fused(gpu):
    print("[fused] drawing the B=1024 K=7 V=151936 workload", flush=True)
    vi, bi = synth.make_fused_inputs()
    t = dict(z=dev(vi.logits), q=dev(vi.draft_probs), d=dev(vi.draft_tokens),
             u=dev(vi.uniforms), L=dev(bi.start_pos), bt=dev(bi.block_table),
             h=dev(bi.target_hidden), hs=dev(bi.h_shared))
    rng = np.random.default_rng(55)
    picks = sorted(set([0, vi.spec.B - 1] + list(rng.choice(vi.spec.B, N_SAMPLED, replace=False))))
    yield vi, bi, t, picks
    del t
    torch.cuda.empty_cache()


def _build(sv, bi, t, out, acc):
    return sv.peagle_build_draft_batch(out, acc, t["d"], t["L"], t["bt"], bi.spec.block_size,
                                       t["h"], t["hs"], bi.mask_token_id)


def _check_build_rows(vi, bi, res, out, acc, picks):
    K = vi.spec.K
    got = {k: (host_bits(v) if k == "hidden" else v.cpu().numpy()) for k, v in res.items()}
    case = dict(out_tokens=out, num_accepted=acc, draft_tokens=vi.draft_tokens,
                start_pos=bi.start_pos, block_table=bi.block_table, block_size=bi.spec.block_size,
                target_hidden=bi.target_hidden, h_shared=bi.h_shared,
                mask_token_id=bi.mask_token_id)
    check_invariants(got, case, K)
    for b in picks:
        one = dict(out_tokens=out[b:b + 1], num_accepted=acc[b:b + 1],
                   draft_tokens=vi.draft_tokens[b:b + 1], start_pos=bi.start_pos[b:b + 1],
                   block_table=bi.block_table[b:b + 1], block_size=bi.spec.block_size,
                   target_hidden=bi.target_hidden[b * (K + 1):(b + 1) * (K + 1)],
                   h_shared=bi.h_shared, mask_token_id=bi.mask_token_id)
        want = oracle.build_draft_batch(**one)
        seg = slice(b * 2 * K, (b + 1) * 2 * K)
        assert np.array_equal(got["input_ids"][seg], want["input_ids"])
        assert np.array_equal(got["positions"][seg], want["positions"])
        assert np.array_equal(got["slot_mapping"][seg], want["slot_mapping"])
        assert np.array_equal(got["hidden"][seg], want["hidden"])
        assert np.array_equal(got["sample_rows"][b] - b * 2 * K, want["sample_rows"][0])


def _well_formed(vi, out, acc):
    K, V = vi.spec.K, vi.spec.V
    assert np.all((acc >= 0) & (acc <= K))
    for b in range(vi.spec.B):
        a = acc[b]
        assert np.array_equal(out[b, :a], vi.draft_tokens[b, :a])
        assert 0 <= out[b, a] < V
        assert np.all(out[b, a + 1:] == -1)


def test_fused_greedy_then_build(gpu, fused):
    vi, bi, t, picks = fused
    out_t, acc_t = gpu.spec_verify_greedy(t["z"], t["d"])
    res = _build(gpu, bi, t, out_t, acc_t)
    torch.cuda.synchronize()
    out, acc = out_t.cpu().numpy(), acc_t.cpu().numpy()
    _well_formed(vi, out, acc)
    for b in picks:
        w_out, w_acc = oracle.verify_greedy(vi.logits[b:b + 1], "bf16", vi.draft_tokens[b:b + 1])
        assert acc[b] == w_acc[0] and np.array_equal(out[b], w_out[0]), b
    _check_build_rows(vi, bi, res, out, acc, picks)


def test_fused_sample_then_build(gpu, fused):
    vi, bi, t, picks = fused
    out_t, acc_t, pd_t = gpu.spec_verify_sample(t["z"], t["q"], t["d"], t["u"], vi.temperature,
                                                want_draft_target_prob=True)
    res = _build(gpu, bi, t, out_t, acc_t)
    torch.cuda.synchronize()
    out, acc, pd = out_t.cpu().numpy(), acc_t.cpu().numpy(), pd_t.cpu().numpy()
    _well_formed(vi, out, acc)
    assert np.all(np.isfinite(pd)) and np.all(pd >= 0) and np.all(pd <= 1)
    for b in picks:
        z64 = oracle.decode_logits(vi.logits[b], "bf16")
        check_sample_sequence(z64, vi.draft_probs[b], vi.draft_tokens[b], vi.uniforms[b],
                              vi.temperature, out[b], acc[b], pd[b])
    _check_build_rows(vi, bi, res, out, acc, picks)
    # acceptance rate of the workload is in the range the drafts are built for
    rate = (acc.sum() / np.minimum(acc + 1, vi.spec.K).sum())
    print(f"[fused] acceptance rate {rate:.3f}, mean accepted {acc.mean():.3f}", flush=True)
    assert 0.3 < rate < 0.8


def test_fused_mixed_then_build(gpu, fused):
    """The same batch as a mixed serving batch: per-sequence temperatures from
    {0, 0.5, 0.7, 1.0, 1.3}, one verify launch sequence, then the build."""
    vi, bi, t, picks = fused
    temps = synth.make_temperatures(vi.spec.B, 15)
    out_t, acc_t, pd_t = gpu.spec_verify_mixed(t["z"], t["q"], t["d"], t["u"], dev(temps),
                                               want_draft_target_prob=True)
    res = _build(gpu, bi, t, out_t, acc_t)
    torch.cuda.synchronize()
    out, acc, pd = out_t.cpu().numpy(), acc_t.cpu().numpy(), pd_t.cpu().numpy()
    _well_formed(vi, out, acc)
    for b in picks:
        z64 = oracle.decode_logits(vi.logits[b], "bf16")
        if temps[b] == 0:
            w_out, w_acc, w_pd = oracle.verify_mixed(vi.logits[b:b + 1], "bf16",
                                                     vi.draft_probs[b:b + 1],
                                                     vi.draft_tokens[b:b + 1],
                                                     vi.uniforms[b:b + 1], temps[b:b + 1])
            assert acc[b] == w_acc[0] and np.array_equal(out[b], w_out[0]), b
            assert np.array_equal(pd[b], w_pd[0].astype(np.float32)), b
        else:
            check_sample_sequence(z64, vi.draft_probs[b], vi.draft_tokens[b], vi.uniforms[b],
                                  float(temps[b]), out[b], acc[b], pd[b])
    _check_build_rows(vi, bi, res, out, acc, picks)


def test_fused_draft_sample(gpu, fused):
    """Drafter-output sampling at the bench shape: the first K logit rows of
    each sequence stand in for the drafter rows, gathered through a row index;
    sampled drafts checked against the oracle."""
    vi, bi, t, picks = fused
    B, K, V = vi.spec.B, vi.spec.K, vi.spec.V
    rows = (np.arange(B, dtype=np.int32)[:, None] * (K + 1) + np.arange(K, dtype=np.int32)).copy()
    u = np.random.default_rng(7).random((B, K), dtype=np.float32)
    tok_t, q_t = gpu.spec_draft_sample(t["z"].view(B * (K + 1), V), K, vi.temperature,
                                       uniforms=dev(u), row_index=dev(rows))
    tok2_t, _ = gpu.spec_draft_sample(t["z"].view(B * (K + 1), V), K, vi.temperature,
                                      uniforms=dev(u), row_index=dev(rows),
                                      want_draft_probs=False)
    torch.cuda.synchronize()
    tok = tok_t.cpu().numpy()
    assert np.array_equal(tok, tok2_t.cpu().numpy())
    assert np.all((tok >= 0) & (tok < V))
    for b in picks:
        qb = q_t[b].cpu().numpy()
        for k in range(K):
            z64 = oracle.decode_logits(vi.logits[b, k], "bf16")
            d, q = oracle.draft.draft_sample_row(z64, float(np.float32(vi.temperature)), u[b, k])
            assert np.allclose(qb[k], q, rtol=1e-5, atol=1e-30), (b, k)
            if tok[b, k] != d:
                assert int(tok[b, k]) in oracle.draft_outcomes(z64, vi.temperature, u[b, k]), (b, k)
