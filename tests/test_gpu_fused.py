"""GPU parity at full size: the fused high-concurrency step.

B=1024 sequences, K=7, V=151936 bf16 logits (2.49 GB) with fp32 draft
probabilities (4.36 GB), verified on the device, then the P-EAGLE batch (H=2048
bf16, prompt lengths U{64..8192}) built from the verify outputs on the same
stream with no host round trip.  Every sequence is compared with the oracle:
the greedy, sampled and mixed verify (decisions within 1e-6 of their threshold
may go either way; those near ties are counted and must stay below 1% of the
decisions), the build bit for bit, every one of the 7168 drafter rows (its q
within 1e-5 relative, its token among the oracle's draws), and the decode
round with q handed over as drafter logits + row descriptors, which also
equals the dense-q round bit for bit.  The oracle runs in worker processes
(tests/fused_oracle.py), each regenerating its sequences from their seeds.
"""
import multiprocessing
import os
import tempfile

import numpy as np
import pytest
import torch

import oracle
import synth
from tests import fused_oracle
from tests.gpu_util import DEV, dev, host_bits
from tests.test_oracle_build import check_invariants

pytestmark = pytest.mark.gpu

CHUNK = 32                 # sequences per oracle task


@pytest.fixture(scope="module")
def fused(gpu):
    print("[fused] drawing the B=1024 K=7 V=151936 workload", flush=True)
    vi, bi = synth.make_fused_inputs()
    t = dict(z=dev(vi.logits), q=dev(vi.draft_probs), d=dev(vi.draft_tokens),
             u=dev(vi.uniforms), L=dev(bi.start_pos), bt=dev(bi.block_table),
             h=dev(bi.target_hidden), hs=dev(bi.h_shared))
    yield vi, bi, t
    del t
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def pool():
    # fresh interpreters that import only numpy, the oracle and the input
    # generator; they never touch the GPU
    p = multiprocessing.get_context("spawn").Pool(min(16, os.cpu_count() or 1))
    yield p
    p.close()
    p.join()


def _chunks(B):
    return [(lo, min(B, lo + CHUNK)) for lo in range(0, B, CHUNK)]


def _run(pool, fn, tasks):
    return pool.map(fn, tasks, chunksize=1)


def _build(sv, bi, t, out, acc):
    return sv.peagle_build_draft_batch(out, acc, t["d"], t["L"], t["bt"], bi.spec.block_size,
                                       t["h"], t["hs"], bi.mask_token_id)


def _check_build_every_row(vi, bi, res, out, acc):
    """The whole build against oracle.build_draft_batch on the GPU's verify
    outputs, bit for bit, plus the batch invariants."""
    got = {k: (host_bits(v) if k == "hidden" else v.cpu().numpy()) for k, v in res.items()}
    case = dict(out_tokens=out, num_accepted=acc, draft_tokens=vi.draft_tokens,
                start_pos=bi.start_pos, block_table=bi.block_table, block_size=bi.spec.block_size,
                target_hidden=bi.target_hidden, h_shared=bi.h_shared,
                mask_token_id=bi.mask_token_id)
    check_invariants(got, case, vi.spec.K)
    want = oracle.build_draft_batch(**case)
    for key in ("input_ids", "positions", "slot_mapping", "hidden", "sample_rows"):
        assert np.array_equal(got[key], want[key]), key


def _check_verify(pool, vi, out, acc, pd, temps=None):
    B, K = vi.spec.B, vi.spec.K
    tasks = [(lo, hi, None if temps is None else temps[lo:hi], out[lo:hi], acc[lo:hi], pd[lo:hi])
             for lo, hi in _chunks(B)]
    res = _run(pool, fused_oracle.verify_task, tasks)
    errors = [e for r in res for e in r[0]]
    flags, aflags = sum(r[1] for r in res), sum(r[2] for r in res)
    assert not errors, errors[:10]
    decisions = B * (K + 1)
    print(f"[fused] every sequence matches the oracle; near ties within 1e-6: {flags} "
          f"({aflags} accept tests, {flags - aflags} final draws) of {decisions} decisions",
          flush=True)
    assert flags <= 0.01 * decisions
    return flags


def test_fused_greedy_every_sequence(gpu, fused, pool):
    """Every sequence of the full batch against the definition of greedy
    verification (numpy's lowest-index argmax chain) and against the oracle."""
    vi, bi, t = fused
    B, K = vi.spec.B, vi.spec.K
    out_t, acc_t = gpu.spec_verify_greedy(t["z"], t["d"])
    torch.cuda.synchronize()
    out, acc = out_t.cpu().numpy(), acc_t.cpu().numpy()
    g = np.empty((B, K + 1), np.int64)
    for lo in range(0, B, 64):
        w = (vi.logits[lo:lo + 64].astype(np.uint32) << np.uint32(16)).view(np.float32)
        g[lo:lo + 64] = np.argmax(w, axis=-1)
    match = vi.draft_tokens == g[:, :K]
    want_a = np.where(match.all(axis=1), K, np.argmin(match, axis=1))
    assert np.array_equal(acc, want_a)
    rows = np.arange(B)
    assert np.array_equal(out[rows, acc], g[rows, acc])
    errors = _run(pool, fused_oracle.greedy_task,
                  [(lo, hi, out[lo:hi], acc[lo:hi]) for lo, hi in _chunks(B)])
    assert not any(errors), [e for r in errors for e in r][:10]


def test_fused_greedy_then_build(gpu, fused):
    vi, bi, t = fused
    out_t, acc_t = gpu.spec_verify_greedy(t["z"], t["d"])
    res = _build(gpu, bi, t, out_t, acc_t)
    torch.cuda.synchronize()
    _check_build_every_row(vi, bi, res, out_t.cpu().numpy(), acc_t.cpu().numpy())


def test_fused_sample_then_build(gpu, fused, pool):
    """The sampled verify of every sequence against the oracle, run to run
    bitwise identical, and the build from its outputs bit for bit."""
    vi, bi, t = fused
    T = vi.temperature
    out_t, acc_t, pd_t = gpu.spec_verify_sample(t["z"], t["q"], t["d"], t["u"], T,
                                                want_draft_target_prob=True)
    res = _build(gpu, bi, t, out_t, acc_t)
    out2, acc2, pd2 = gpu.spec_verify_sample(t["z"], t["q"], t["d"], t["u"], T,
                                             want_draft_target_prob=True)
    torch.cuda.synchronize()
    assert torch.equal(out_t, out2) and torch.equal(acc_t, acc2)
    assert torch.equal(pd_t.view(torch.int32), pd2.view(torch.int32))
    out, acc, pd = out_t.cpu().numpy(), acc_t.cpu().numpy(), pd_t.cpu().numpy()
    _check_verify(pool, vi, out, acc, pd)
    _check_build_every_row(vi, bi, res, out, acc)
    rate = (acc.sum() / np.minimum(acc + 1, vi.spec.K).sum())
    print(f"[fused] acceptance rate {rate:.3f}, mean accepted {acc.mean():.3f}", flush=True)
    assert 0.3 < rate < 0.8


def test_fused_mixed_then_build(gpu, fused, pool):
    """The same batch as a mixed serving batch: per-sequence temperatures from
    {0, 0.5, 0.7, 1.0, 1.3}, one verify launch sequence, then the build; every
    sequence against the oracle (greedy ones exactly)."""
    vi, bi, t = fused
    temps = synth.make_temperatures(vi.spec.B, 15)
    out_t, acc_t, pd_t = gpu.spec_verify_mixed(t["z"], t["q"], t["d"], t["u"], dev(temps),
                                               want_draft_target_prob=True)
    res = _build(gpu, bi, t, out_t, acc_t)
    torch.cuda.synchronize()
    out, acc, pd = out_t.cpu().numpy(), acc_t.cpu().numpy(), pd_t.cpu().numpy()
    assert (temps == 0).sum() > 100 and (temps > 0).sum() > 500
    _check_verify(pool, vi, out, acc, pd, temps=temps)
    _check_build_every_row(vi, bi, res, out, acc)


def test_fused_draft_sample(gpu, fused, pool):
    """Drafter-output sampling at the bench shape: the first K logit rows of
    each sequence stand in for the drafter rows, gathered through a row index;
    all 7168 rows against the oracle (q and token)."""
    vi, bi, t = fused
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
    shm = "/dev/shm" if os.path.isdir("/dev/shm") else None
    with tempfile.TemporaryDirectory(dir=shm) as d:
        path = os.path.join(d, "q.npy")
        np.save(path, q_t.cpu().numpy())
        del q_t
        Td = float(np.float32(vi.temperature))
        errors = _run(pool, fused_oracle.draft_task,
                      [(lo, hi, Td, u[lo:hi], tok[lo:hi], path) for lo, hi in _chunks(B)])
    assert not any(errors), [e for r in errors for e in r][:10]


def test_fused_lq_round(gpu, fused, pool):
    """A decode round at the bench shape with the drafter's q handed over as
    logits + row descriptors: drafter sampling (the first K logit rows of each
    sequence gathered through a row index, T = 0.7), then the verify from
    drafter logits, which equals the dense-q verify for every sequence bit for
    bit; every sequence against the oracle (q from the oracle's drafter
    softmax, drafts from the oracle's drafter sampler)."""
    vi, bi, t = fused
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
    res = _run(pool, fused_oracle.lq_task,
               [(lo, hi, vi.temperature, ud[lo:hi], tok[lo:hi], out[lo:hi], acc[lo:hi], pd[lo:hi])
                for lo, hi in _chunks(B)])
    errors = [e for r in res for e in r[0]]
    compared = sum(r[1] for r in res)
    assert not errors, errors[:10]
    print(f"[fused] decode round: {compared} of {B} sequences compared with the oracle "
          f"(the rest drafted a near tie of the drafter's own draw)", flush=True)
    assert compared >= B - 16
