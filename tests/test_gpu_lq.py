"""GPU: the sampled verify that recomputes q from the drafter logits.

spec_draft_sample writes, for each drafted row, the dense q and the row
descriptor; spec_verify_sample on the dense q and spec_verify_sample_lq on
the drafter logits + descriptors must then agree bit for bit (tokens, accept
counts, p_k(d_k)).  The lq results are also checked against the oracle: q from
oracle.draft.draft_probs, then the sampled-verify oracle with its near-tie
tolerance.  Covered: the 151936-token bf16 shape; a ragged bf16 vocabulary
with drafter rows gathered through a row index, greedy-drafted sequences and
invalid drafter rows; fp32 logits at a vocabulary that is a multiple of 8 and
one that is not (rows gathered through a row index); no drafts at all;
mixed serving batches (spec_verify_mixed_lq against spec_verify_mixed on the
dense q and against the oracle); and the vocabularies of the shape sweep
around multiples of the CDF tile, uniform and mixed.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.workloads import DRAFT_CONFIGS, make_draft_inputs
from tests.gpu_util import DEV, check_sample_sequence, dev
from tests.test_gpu_shapes import VOCABS

pytestmark = pytest.mark.gpu


def _chain(sv, z, zd, K, Td, T, u_draft, u_verify, rows=None, temps=None):
    tok, q, desc = sv.spec_draft_sample(zd, K, Td, uniforms=u_draft, row_index=rows,
                                        temperatures=temps, want_row_desc=True)
    dense = sv.spec_verify_sample(z, q, tok, u_verify, T, want_draft_target_prob=True)
    lq = sv.spec_verify_sample_lq(z, zd, desc, tok, u_verify, T, drafter_rows=rows,
                                  want_draft_target_prob=True)
    torch.cuda.synchronize()
    return tok, q, desc, dense, lq


def _same(dense, lq):
    assert torch.equal(dense[0], lq[0]) and torch.equal(dense[1], lq[1])
    assert torch.equal(dense[2].view(torch.int32), lq[2].view(torch.int32))


def test_lq_matches_dense_and_oracle_large_vocab(gpu):
    vi = synth.make_verify_inputs(synth.verify_config(5), seqs=range(48))
    di = make_draft_inputs(DRAFT_CONFIGS["draft-mid"])           # B=48, K=7, V=151936 bf16
    B, K, V = 48, 7, 151936
    tok, q, desc, dense, lq = _chain(gpu, dev(vi.logits), dev(di.logits), K, di.temperature,
                                     vi.temperature, dev(di.uniforms), dev(vi.uniforms))
    _same(dense, lq)
    out, acc, pd = (x.cpu().numpy() for x in lq)
    tok = tok.cpu().numpy()
    oq = oracle.draft.draft_probs(di.logits, "bf16", di.temperature, B, K)
    checked = 0
    for b in range(B):
        od = [oracle.draft.draft_sample_row(oracle.decode_logits(di.logits[b * K + k], "bf16"),
                                            float(np.float32(di.temperature)), di.uniforms[b, k])[0]
              for k in range(K)]
        if list(tok[b]) != od:
            continue                      # a flagged near tie in the draft itself
        z64 = oracle.decode_logits(vi.logits[b], "bf16")
        check_sample_sequence(z64, oq[b], tok[b], vi.uniforms[b], vi.temperature, out[b], acc[b],
                              pd[b])
        checked += 1
    assert checked >= B - 2


def test_lq_gathered_rows_greedy_drafts_and_bad_rows(gpu):
    di = make_draft_inputs(DRAFT_CONFIGS["draft-ragged"])         # fp32-free: bf16, V=30011
    s = di.spec
    B, K, V = s.B, s.K, s.V
    rng = np.random.default_rng(91)
    z = synth.f32_to_bf16_bits((3.0 * rng.standard_normal((B, K + 1, V))).astype(np.float32))
    uv = rng.random((B, K + 1), dtype=np.float32)
    temps = di.temperatures.copy()
    temps[0] = 0.0                                                # a greedy-drafted sequence
    tok, q, desc, dense, lq = _chain(gpu, dev(z), dev(di.logits), K, s.temperature, 0.9,
                                     dev(di.uniforms), dev(uv), rows=dev(di.row_index),
                                     temps=dev(temps))
    _same(dense, lq)
    d = desc.cpu().numpy()
    assert np.all(d[0, :, 0] == 0) and np.all(d[0, :, 3] == tok.cpu().numpy()[0])
    # a drafter row outside the logits: flagged, and counted as q = 0 (the
    # dense path sees the all-zero q row that spec_draft_sample writes for it)
    rows = di.row_index.copy()
    rows[2, 1] = B * s.rows_per_seq + 3
    err_d = torch.zeros(1, dtype=torch.int32, device=DEV)
    err_v = torch.zeros(1, dtype=torch.int32, device=DEV)
    tok2, q2, desc2 = gpu.spec_draft_sample(dev(di.logits), K, s.temperature,
                                            uniforms=dev(di.uniforms), row_index=dev(rows),
                                            temperatures=dev(temps), want_row_desc=True,
                                            device_error=err_d)
    tok2[2, 1] = 5                                                # a valid token for the test
    a1 = gpu.spec_verify_sample(dev(z), q2, tok2, dev(uv), 0.9, want_draft_target_prob=True)
    a2 = gpu.spec_verify_sample_lq(dev(z), dev(di.logits), desc2, tok2, dev(uv), 0.9,
                                   drafter_rows=dev(rows), want_draft_target_prob=True,
                                   device_error=err_v)
    torch.cuda.synchronize()
    assert int(err_d.item()) == gpu.DEVERR_ROW_INDEX
    assert int(err_v.item()) == gpu.DEVERR_ROW_INDEX
    _same(a1, a2)


@pytest.mark.parametrize("V", [4096, 1001])
def test_lq_fp32(gpu, V):
    B, K, R = 6, 4, 40
    rng = np.random.default_rng(93 + V)
    z = (2.5 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    # drafter rows: the target rows plus noise, stored in shuffled order
    rows = rng.permutation(R)[:B * K].reshape(B, K).astype(np.int32)
    zd = (2.5 * rng.standard_normal((R, V))).astype(np.float32)
    zd[rows] = z[:, :K] + rng.standard_normal((B, K, V)).astype(np.float32)
    ud = rng.random((B, K), dtype=np.float32)
    uv = rng.random((B, K + 1), dtype=np.float32)
    Td, T = 1.1, 0.8
    tok, q, desc, dense, lq = _chain(gpu, dev(z), dev(zd), K, Td, T, dev(ud), dev(uv),
                                     rows=dev(rows))
    _same(dense, lq)
    out, acc, pd = (x.cpu().numpy() for x in lq)
    tok = tok.cpu().numpy()
    oq = oracle.draft.draft_probs(zd, "f32", Td, B, K, row_index=rows)
    checked = 0
    for b in range(B):
        od = [oracle.draft.draft_sample_row(zd[rows[b, k]].astype(np.float64),
                                            float(np.float32(Td)), ud[b, k])[0]
              for k in range(K)]
        if list(tok[b]) != od:
            continue                      # a flagged near tie in the draft itself
        check_sample_sequence(z[b].astype(np.float64), oq[b], tok[b], uv[b], float(np.float32(T)),
                              out[b], acc[b], pd[b])
        checked += 1
    assert checked >= B - 1


def test_lq_without_drafts(gpu):
    z = dev((2.0 * np.random.default_rng(3).standard_normal((3, 1, 64))).astype(np.float32))
    u = dev(np.random.default_rng(4).random((3, 1), dtype=np.float32))
    zd = torch.zeros((0, 64), dtype=torch.float32, device=DEV)
    desc = torch.zeros((3, 0, 4), dtype=torch.int32, device=DEV)
    d = torch.zeros((3, 0), dtype=torch.int32, device=DEV)
    o1, a1, _ = gpu.spec_verify_sample_lq(z, zd, desc, d, u, 1.0)
    o2, a2, _ = gpu.spec_verify_sample(z, torch.zeros((3, 0, 64), device=DEV), d, u, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(a1, a2)


@pytest.mark.parametrize("dtype,V,B", [("bf16", 40000, 300), ("f32", 40001, 300),
                                        ("bf16", 40000, 256), ("f32", 40001, 700)])
def test_lq_matches_dense_mid_batch(gpu, dtype, V, B):
    """Mid-size batches with rows of more than 16 CDF tiles, one draw
    workgroup per sequence which searches the token itself (1024 threads at
    B = 256, 512 at B = 300, 256 at B = 700): the drafter-logit verify equals
    the dense-q verify bit for bit."""
    K = 3
    rng = np.random.default_rng(V + B)
    z = (3 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    zd = (3 * rng.standard_normal((B * K, V))).astype(np.float32)
    if dtype == "bf16":
        z, zd = synth.f32_to_bf16_bits(z), synth.f32_to_bf16_bits(zd)
    ud = rng.random((B, K), dtype=np.float32)
    uv = rng.random((B, K + 1), dtype=np.float32)
    _, _, _, dense, lq = _chain(gpu, dev(z), dev(zd), K, 0.8, 0.9, dev(ud), dev(uv))
    _same(dense, lq)


@pytest.mark.parametrize("dtype,V,B", [("bf16", 151936, 24), ("bf16", 32000, 40),
                                       ("f32", 4099, 40)])
def test_mixed_lq_matches_mixed_and_oracle(gpu, dtype, V, B):
    """A mixed serving batch (target temperatures per sequence from {0, 0.5,
    0.7, 1.0, 1.3}) drafted at per-sequence drafter temperatures (greedy
    drafting included): spec_verify_mixed on the dense q and
    spec_verify_mixed_lq on the drafter logits + descriptors agree bit for
    bit, and every sequence matches the oracle (greedy ones exactly)."""
    K = 5
    rng = np.random.default_rng(V + B)
    z = (3.0 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    z[:, :, :8] += 6.0
    zd = (z[:, :K] + rng.standard_normal((B, K, V)).astype(np.float32)).reshape(B * K, V)
    if dtype == "bf16":
        z, zd = synth.f32_to_bf16_bits(z), synth.f32_to_bf16_bits(zd)
    temps_d = synth.make_temperatures(B, 71)
    temps_v = synth.make_temperatures(B, 72)
    assert (temps_v == 0).any() and (temps_v > 0).any() and (temps_d == 0).any()
    ud = rng.random((B, K), dtype=np.float32)
    uv = rng.random((B, K + 1), dtype=np.float32)
    tok, q, desc = gpu.spec_draft_sample(dev(zd), K, 1.0, uniforms=dev(ud),
                                         temperatures=dev(temps_d), want_row_desc=True)
    dense = gpu.spec_verify_mixed(dev(z), q, tok, dev(uv), dev(temps_v),
                                  want_draft_target_prob=True)
    lq = gpu.spec_verify_mixed_lq(dev(z), dev(zd), desc, tok, dev(uv), dev(temps_v),
                                  want_draft_target_prob=True)
    torch.cuda.synchronize()
    _same(dense, lq)
    out, acc, pd = (x.cpu().numpy() for x in lq)
    tok = tok.cpu().numpy()
    oq = oracle.draft.draft_probs(zd, dtype, 1.0, B, K, temperatures=temps_d)
    checked = mism = flags = 0
    for b in range(B):
        od = [oracle.draft.draft_sample_row(oracle.decode_logits(zd[b * K + k], dtype),
                                            float(temps_d[b]), ud[b, k])[0] for k in range(K)]
        if list(tok[b]) != od:
            continue                      # a flagged near tie in the draft itself
        z64 = oracle.decode_logits(z[b], dtype)
        if oracle.mixed.is_greedy(temps_v[b]):
            w_out, w_acc, w_pd = oracle.verify_mixed(z[b:b + 1], dtype, oq[b:b + 1],
                                                     tok[b:b + 1], uv[b:b + 1],
                                                     temps_v[b:b + 1])
            assert acc[b] == w_acc[0] and np.array_equal(out[b], w_out[0]), b
            assert np.array_equal(pd[b], w_pd[0].astype(np.float32)), b
        else:
            same, f = check_sample_sequence(z64, oq[b], tok[b], uv[b], float(temps_v[b]), out[b],
                                            acc[b], pd[b])
            mism += not same
            flags += f
        checked += 1
    assert mism <= flags
    assert checked >= B - 2


@pytest.mark.parametrize("i", range(len(VOCABS)))
def test_lq_boundary_shapes(gpu, i):
    """q from the drafter logits over the vocabularies of the shape sweep
    (just below, at and just above multiples of the 2048-element CDF tile),
    with random B and K, both dtypes, and uniform and mixed temperatures in
    turn, so that every draw form (tiles in registers, one workgroup per
    sequence, chunks with the locate kernel) meets the drafter-logit loads:
    bit for bit the dense verify on the same drafting, and every sequence
    against the oracle (q from oracle.draft.draft_probs)."""
    rng = np.random.default_rng(9100 + i)
    V = VOCABS[i]
    B = int(rng.integers(1, 24))
    K = int(rng.integers(1, 10))
    dtype = ("bf16", "f32")[i % 2]
    mixed = i % 3 == 0
    z = (3.0 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    z[:, :, :8] += 6.0
    zd = (z[:, :K] + rng.standard_normal((B, K, V)).astype(np.float32)).reshape(B * K, V)
    if dtype == "bf16":
        z, zd = synth.f32_to_bf16_bits(z), synth.f32_to_bf16_bits(zd)
    ud = rng.random((B, K), dtype=np.float32)
    uv = rng.random((B, K + 1), dtype=np.float32)
    Td, T = 0.8, 0.9
    temps_d = synth.make_temperatures(B, 7 + i) if mixed else None
    temps_v = synth.make_temperatures(B, 17 + i) if mixed else None
    tok, q, desc = gpu.spec_draft_sample(dev(zd), K, Td, uniforms=dev(ud),
                                         temperatures=None if temps_d is None else dev(temps_d),
                                         want_row_desc=True)
    if mixed:
        dense = gpu.spec_verify_mixed(dev(z), q, tok, dev(uv), dev(temps_v),
                                      want_draft_target_prob=True)
        lq = gpu.spec_verify_mixed_lq(dev(z), dev(zd), desc, tok, dev(uv), dev(temps_v),
                                      want_draft_target_prob=True)
    else:
        dense = gpu.spec_verify_sample(dev(z), q, tok, dev(uv), T, want_draft_target_prob=True)
        lq = gpu.spec_verify_sample_lq(dev(z), dev(zd), desc, tok, dev(uv), T,
                                       want_draft_target_prob=True)
    torch.cuda.synchronize()
    _same(dense, lq)
    out, acc, pd = (x.cpu().numpy() for x in lq)
    tok = tok.cpu().numpy()
    oq = oracle.draft.draft_probs(zd, dtype, Td, B, K, temperatures=temps_d)
    for b in range(B):
        z64 = oracle.decode_logits(z[b], dtype)
        if mixed and oracle.mixed.is_greedy(temps_v[b]):
            w_out, w_acc, w_pd = oracle.verify_mixed(z[b:b + 1], dtype, oq[b:b + 1], tok[b:b + 1],
                                                     uv[b:b + 1], temps_v[b:b + 1])
            assert acc[b] == w_acc[0] and np.array_equal(out[b], w_out[0]), b
            assert np.array_equal(pd[b], w_pd[0].astype(np.float32)), b
        else:
            Tb = float(temps_v[b]) if mixed else T
            check_sample_sequence(z64, oq[b], tok[b], uv[b], Tb, out[b], acc[b], pd[b])
