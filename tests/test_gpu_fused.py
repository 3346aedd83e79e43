"""GPU parity at full size: the fused high-concurrency step.

B=1024 sequences, K=7, V=151936 bf16 logits (2.49 GB) with fp32 draft
probabilities (4.36 GB), verified on the device, then the P-EAGLE batch (H=2048
bf16, prompt lengths U{64..8192}) built from the verify outputs on the same
stream with no host round trip.  Every sequence is checked for well-formed
output and the build invariants; a seeded sample of sequences is checked
against the oracle one by one (the oracle's cost limits the sample), and every
sequence against the greedy definition (numpy argmax chain) and against
properties of rejection sampling (each accept test, the drawn token in the
support of its distribution).  The decode round with the drafter's q handed
over as drafter logits + row descriptors is checked against the dense-q round
bit for bit on every sequence.
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


def _widened(vi, lo, hi):
    """Logit rows of sequences lo..hi-1 as float32 (bf16 widened exactly)."""
    return (vi.logits[lo:hi].astype(np.uint32) << np.uint32(16)).view(np.float32)


def _all_row_argmax(vi, chunk=64):
    """Lowest-index argmax of every logit row of the batch, [B][K+1]."""
    B = vi.spec.B
    g = np.empty((B, vi.spec.K + 1), np.int64)
    for lo in range(0, B, chunk):
        g[lo:lo + chunk] = np.argmax(_widened(vi, lo, min(B, lo + chunk)), axis=-1)
    return g


def test_fused_greedy_every_sequence(gpu, fused):
    """Every sequence of the full batch against the definition of greedy
    verification: drafts accepted while each equals its row's lowest-index
    argmax (numpy), then the argmax of the first mismatching row (or of row K)."""
    vi, bi, t, picks = fused
    B, K = vi.spec.B, vi.spec.K
    out_t, acc_t = gpu.spec_verify_greedy(t["z"], t["d"])
    torch.cuda.synchronize()
    out, acc = out_t.cpu().numpy(), acc_t.cpu().numpy()
    g = _all_row_argmax(vi)
    match = vi.draft_tokens == g[:, :K]
    want_a = np.where(match.all(axis=1), K, np.argmin(match, axis=1))
    assert np.array_equal(acc, want_a)
    rows = np.arange(B)
    assert np.array_equal(out[rows, acc], g[rows, acc])
    _well_formed(vi, out, acc)


def test_fused_sample_every_sequence(gpu, fused):
    """Every sequence of the full batch against properties of rejection
    sampling that hold at any size, with p computed here in fp64 from each
    row's max and sum of exponentials: draft k < a passed its test u_k <
    p_k(d_k) / q_k(d_k) and draft a (a < K) failed it, except where u_k lies
    within 1e-5 (relative) of the ratio; the new token lies in the support of
    the distribution it was drawn from: max(0, p_a - q_a) for a < K (p_a(c) >
    q_a(c), up to the fp32 rounding of p), p_K for a = K."""
    vi, bi, t, picks = fused
    B, K, T = vi.spec.B, vi.spec.K, vi.temperature
    out_t, acc_t, pd_t = gpu.spec_verify_sample(t["z"], t["q"], t["d"], t["u"], T,
                                                want_draft_target_prob=True)
    out2, acc2, pd2 = gpu.spec_verify_sample(t["z"], t["q"], t["d"], t["u"], T,
                                             want_draft_target_prob=True)
    torch.cuda.synchronize()
    # run to run: bitwise identical (no floating-point atomics anywhere)
    assert torch.equal(out_t, out2) and torch.equal(acc_t, acc2)
    assert torch.equal(pd_t.view(torch.int32), pd2.view(torch.int32))
    out, acc = out_t.cpu().numpy(), acc_t.cpu().numpy()
    _well_formed(vi, out, acc)
    rows = np.arange(B)
    c = out[rows, acc]
    d, u = vi.draft_tokens, vi.uniforms.astype(np.float64)
    p_d = np.empty((B, K))          # p_k(d_k)
    p_c = np.empty(B)               # p_a(c)
    chunk = 32
    for lo in range(0, B, chunk):
        hi = min(B, lo + chunk)
        z = _widened(vi, lo, hi).astype(np.float64)            # [n][K+1][V]
        m = z.max(axis=-1, keepdims=True)
        lse = np.log(np.exp((z - m) / T).sum(axis=-1))          # [n][K+1]
        n = np.arange(hi - lo)
        zd = z[n[:, None], np.arange(K)[None, :], d[lo:hi]]
        p_d[lo:hi] = np.exp((zd - m[:, :K, 0]) / T - lse[:, :K])
        a = acc[lo:hi]
        p_c[lo:hi] = np.exp((z[n, a, c[lo:hi]] - m[n, a, 0]) / T - lse[n, a])
    q_d = np.take_along_axis(vi.draft_probs, d[:, :, None].astype(np.int64), axis=2)[:, :, 0]
    q_d = q_d.astype(np.float64)
    ratio = np.where(q_d > 0, p_d / np.where(q_d > 0, q_d, 1.0), np.where(p_d > 0, np.inf, 0.0))
    passed = u[:, :K] < ratio
    near = np.abs(u[:, :K] - ratio) <= 1e-5 * np.maximum(1.0, ratio)
    k = np.arange(K)[None, :]
    must_pass = k < acc[:, None]
    must_fail = k == acc[:, None]
    bad = (must_pass & ~passed & ~near) | (must_fail & passed & ~near)
    assert not bad.any(), np.argwhere(bad)[:10]
    rej = acc < K
    q_c = vi.draft_probs[rows[rej], acc[rej], c[rej]].astype(np.float64)
    assert np.all(p_c[rej] > q_c * (1 - 1e-5)), np.flatnonzero(rej)[p_c[rej] <= q_c * (1 - 1e-5)]
    assert np.all(p_c[~rej] > 0)
    print(f"[fused] {int(near.sum())} accept tests within 1e-5 of their ratio", flush=True)


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


def test_fused_lq_round(gpu, fused):
    """A decode round at the bench shape with the drafter's q handed over as
    logits + row descriptors: drafter sampling (the first K logit rows of each
    sequence gathered through a row index, T = 0.7), then the verify from
    drafter logits, which equals the dense-q verify for every sequence bit for
    bit; sampled sequences checked against the oracle (q from the oracle's
    drafter softmax, drafts from the oracle's drafter sampler)."""
    vi, bi, t, picks = fused
    B, K, V = vi.spec.B, vi.spec.K, vi.spec.V
    rows = (np.arange(B, dtype=np.int32)[:, None] * (K + 1) + np.arange(K, dtype=np.int32)).copy()
    ud = np.random.default_rng(7).random((B, K), dtype=np.float32)
    zd, rows_t = t["z"].view(B * (K + 1), V), dev(rows)
    tok_t, q_t, desc_t = gpu.spec_draft_sample(zd, K, vi.temperature, uniforms=dev(ud),
                                               row_index=rows_t, want_row_desc=True)
    dense = gpu.spec_verify_sample(t["z"], q_t, tok_t, t["u"], vi.temperature,
                                   want_draft_target_prob=True)
    del q_t
    lq = gpu.spec_verify_sample_lq(t["z"], zd, desc_t, tok_t, t["u"], vi.temperature,
                                   drafter_rows=rows_t, want_draft_target_prob=True)
    torch.cuda.synchronize()
    assert torch.equal(dense[0], lq[0]) and torch.equal(dense[1], lq[1])
    assert torch.equal(dense[2].view(torch.int32), lq[2].view(torch.int32))
    tok = tok_t.cpu().numpy()
    out, acc, pd = (x.cpu().numpy() for x in lq)
    assert np.all((acc >= 0) & (acc <= K))
    for b in range(B):
        a = acc[b]
        assert np.array_equal(out[b, :a], tok[b, :a]) and 0 <= out[b, a] < V
        assert np.all(out[b, a + 1:] == -1)
    Td = float(np.float32(vi.temperature))
    checked = 0
    for b in picks:
        zq = [oracle.decode_logits(vi.logits[b, k], "bf16") for k in range(K)]
        drafted = [oracle.draft.draft_sample_row(zq[k], Td, ud[b, k]) for k in range(K)]
        od = np.array([x[0] for x in drafted], np.int32)
        if not np.array_equal(tok[b], od):
            continue                      # a flagged near tie in the draft itself
        oq = np.stack([x[1] for x in drafted])
        check_sample_sequence(oracle.decode_logits(vi.logits[b], "bf16"), oq, od, vi.uniforms[b],
                              vi.temperature, out[b], acc[b], pd[b])
        checked += 1
    assert checked >= len(picks) - 1
