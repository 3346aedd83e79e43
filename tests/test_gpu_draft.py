"""GPU parity: spec_draft_sample against the drafter-sampling oracle.

Draft probabilities within 1e-5 relative (absolute floor 1e-30); a draft token
must be the oracle's, or, when u * S lies within 1e-6 of a CDF boundary, one of
the tokens the oracle lists for that near tie (oracle.draft_outcomes); greedy
rows (T = 0) exactly.  Covered: the three drafter workloads (fp32, ragged bf16
with a row gather and mixed per-sequence temperatures, 151936-token bf16),
ragged vocabularies across tile boundaries up to the maximum, ties, -inf
logits, invalid row indices and temperatures, the q-less variant,
determinism, a chi-square test of the GPU's own draws, and drafting followed
by the verify on the GPU.
"""
import numpy as np
import pytest
import torch
from scipy import stats

import oracle
import synth
from synth.workloads import DRAFT_CONFIGS, make_draft_inputs
from tests.gpu_util import DEV, P_ATOL, P_RTOL, TIE_TOL, check_sample_sequence, dev

pytestmark = pytest.mark.gpu


def _rows(B, K, row_index):
    return np.arange(B * K).reshape(B, K) if row_index is None else row_index


def _temps(B, T, temps):
    return np.full(B, np.float32(T)) if temps is None else temps


def _parity(sv, logits, dtype, u, T, B, K, row_index=None, temps=None, want_q=True,
            max_flag_frac=0.01):
    tok, q = sv.spec_draft_sample(dev(logits), K, T, uniforms=None if u is None else dev(u),
                                  row_index=None if row_index is None else dev(row_index),
                                  temperatures=None if temps is None else dev(temps),
                                  want_draft_probs=want_q)
    torch.cuda.synchronize()
    tok = tok.cpu().numpy()
    q = q.cpu().numpy() if want_q else None
    rows = _rows(B, K, row_index)
    Ts = _temps(B, T, temps)
    flags = 0
    for b in range(B):
        for k in range(K):
            z = oracle.decode_logits(logits[rows[b, k]], dtype)
            Tb = float(Ts[b])
            uk = 0.0 if u is None else float(u[b, k])
            want_d, oq = oracle.draft.draft_sample_row(z, Tb, uk)
            if q is not None:
                assert np.allclose(q[b, k], oq, rtol=P_RTOL, atol=P_ATOL), (b, k)
            if tok[b, k] != want_d:
                allowed = oracle.draft_outcomes(z, Tb, uk, tol=TIE_TOL)
                assert int(tok[b, k]) in allowed, (b, k, tok[b, k], want_d, allowed)
                flags += 1
    assert flags <= max(2, max_flag_frac * B * K)
    return tok, q


@pytest.mark.parametrize("name", ["draft-tiny", "draft-ragged", "draft-mid"])
def test_draft_workloads(gpu, name):
    di = make_draft_inputs(DRAFT_CONFIGS[name])
    s = di.spec
    _parity(gpu, di.logits, s.dtype, di.uniforms, s.temperature, s.B, s.K, di.row_index,
            di.temperatures)


@pytest.mark.parametrize("V,dtype", [(1, "f32"), (7, "bf16"), (2047, "f32"), (2049, "bf16"),
                                     (4096, "bf16"), (30000, "f32"), (1 << 19, "bf16")])
def test_ragged_vocabularies(gpu, V, dtype):
    rng = np.random.default_rng(V)
    B, K = 2, 3
    z = (3.0 * rng.standard_normal((B * K, V))).astype(np.float32)
    if V > 3:
        z[:, rng.integers(0, V, size=3)] = -np.inf
    logits = synth.f32_to_bf16_bits(z) if dtype == "bf16" else z
    u = rng.random((B, K), dtype=np.float32)
    tok, _ = _parity(gpu, logits, dtype, u, 0.8, B, K)
    # the tokens-only kernel (no q written) draws the same tokens
    tok2, _ = _parity(gpu, logits, dtype, u, 0.8, B, K, want_q=False)
    assert np.array_equal(tok, tok2)


@pytest.mark.parametrize("V", [5000, 40000])
def test_greedy_drafting_ties_and_no_uniforms(gpu, V):
    # V = 40000 (fp32): long enough for the row statistics' wave-block loop
    rng = np.random.default_rng(3)
    B, K = 3, 4
    z = rng.standard_normal((B * K, V)).astype(np.float32)
    for r in range(B * K):                 # ties at the max, across octets and tiles
        idx = rng.choice(V, size=3, replace=False)
        z[r, idx] = 10.0
    tok, q = _parity(gpu, z, "f32", None, 0.0, B, K)
    assert np.all(q.sum(axis=2) == 1.0) and np.all(q.max(axis=2) == 1.0)
    tok2, _ = _parity(gpu, z, "f32", None, 0.0, B, K, want_q=False)
    assert np.array_equal(tok, tok2)


def test_invalid_rows_and_temperatures(gpu):
    rng = np.random.default_rng(4)
    B, K, V = 4, 2, 600
    z = rng.standard_normal((10, V)).astype(np.float32)
    rows = np.array([[0, 1], [2, -1], [10, 3], [4, 5]], dtype=np.int32)
    temps = np.array([0.7, 1.0, -1.0, np.nan], dtype=np.float32)
    u = rng.random((B, K), dtype=np.float32)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    tok, q = gpu.spec_draft_sample(dev(z), K, 1.0, uniforms=dev(u), row_index=dev(rows),
                                   temperatures=dev(temps), device_error=err)
    torch.cuda.synchronize()
    tok, q = tok.cpu().numpy(), q.cpu().numpy()
    assert int(err.item()) == gpu.DEVERR_ROW_INDEX | gpu.DEVERR_TEMPERATURE
    for b, k in [(1, 1), (2, 0)]:
        assert tok[b, k] == -1 and not q[b, k].any()
    # bad temperatures are treated as greedy
    for b, k in [(2, 1), (3, 0), (3, 1)]:
        zr = z[rows[b, k]].astype(np.float64)
        assert tok[b, k] == oracle.first_argmax(zr)
        assert q[b, k, tok[b, k]] == 1.0 and q[b, k].sum() == 1.0
    # the good rows are unaffected
    for b, k in [(0, 0), (0, 1), (1, 0)]:
        zr = z[rows[b, k]].astype(np.float64)
        assert int(tok[b, k]) in oracle.draft_outcomes(zr, float(temps[b]), float(u[b, k]))


def test_without_probs_and_determinism(gpu):
    di = make_draft_inputs(DRAFT_CONFIGS["draft-ragged"])
    s = di.spec
    args = (dev(di.logits), s.K, s.temperature)
    kw = dict(uniforms=dev(di.uniforms), row_index=dev(di.row_index),
              temperatures=dev(di.temperatures))
    t1, q1 = gpu.spec_draft_sample(*args, **kw)
    t2, q2 = gpu.spec_draft_sample(*args, **kw)
    t3, q3 = gpu.spec_draft_sample(*args, want_draft_probs=False, **kw)
    torch.cuda.synchronize()
    assert q3 is None
    assert torch.equal(t1, t2) and torch.equal(t1, t3)
    assert torch.equal(q1.view(torch.int32), q2.view(torch.int32))


def test_empty_batch(gpu):
    z = torch.zeros((0, 16), dtype=torch.float32, device=DEV)
    tok, q = gpu.spec_draft_sample(z, 3, 0.7, uniforms=torch.zeros((0, 3), device=DEV))
    assert tok.shape == (0, 3) and q.shape == (0, 3, 16)


def test_gpu_draws_follow_q(gpu):
    """One drafter row gathered N times with fresh uniforms: the GPU's draws
    follow the oracle's q (chi-square, df = V - 1)."""
    rng = np.random.default_rng(12)
    V, N, T = 48, 60_000, 0.9
    z = (2.0 * rng.standard_normal((1, V))).astype(np.float32)
    z[0, 5] = -np.inf
    rows = np.zeros((N, 1), dtype=np.int32)
    u = rng.random((N, 1), dtype=np.float32)
    tok, _ = gpu.spec_draft_sample(dev(z), 1, T, uniforms=dev(u), row_index=dev(rows),
                                   want_draft_probs=False)
    counts = np.bincount(tok.cpu().numpy()[:, 0], minlength=V)
    q = oracle.draft.draft_distribution(z[0].astype(np.float64), T)
    assert counts[5] == 0
    obs, exp = counts[q > 0], q[q > 0] * N
    small = exp < 5                        # pool cells with small expectation
    obs = np.concatenate([obs[~small], [obs[small].sum()]])
    exp = np.concatenate([exp[~small], [exp[small].sum()]])
    assert stats.chisquare(obs, exp).pvalue > 1e-4


def test_draft_then_verify_on_gpu(gpu):
    """Drafts and q from the GPU drafter feed the GPU verify.  The oracle
    drafts from the same seeded drafter rows and uniforms and verifies its own
    drafts; the GPU chain must reach an outcome the oracle accepts (sequences
    whose GPU draft was a flagged near tie are skipped)."""
    vi = synth.make_verify_inputs(synth.verify_config(2))
    B, K, V = vi.spec.B, vi.spec.K, vi.spec.V
    rng = np.random.default_rng(21)
    zd = (vi.logits[:, :K] + rng.standard_normal((B, K, V)).astype(np.float32)).reshape(B * K, V)
    u = rng.random((B, K), dtype=np.float32)
    d, q = gpu.spec_draft_sample(dev(zd), K, vi.temperature, uniforms=dev(u))
    out, acc, pd = gpu.spec_verify_sample(dev(vi.logits), q, d, dev(vi.uniforms), vi.temperature,
                                          want_draft_target_prob=True)
    torch.cuda.synchronize()
    d = d.cpu().numpy()
    out, acc, pd = out.cpu().numpy(), acc.cpu().numpy(), pd.cpu().numpy()
    od, oq = oracle.draft_sample(zd, "f32", u, vi.temperature, B, K)
    oq32 = oq.astype(np.float32)
    checked = 0
    for b in range(B):
        if not np.array_equal(d[b], od[b]):
            continue
        z64 = oracle.decode_logits(vi.logits[b], vi.spec.dtype)
        check_sample_sequence(z64, oq32[b], od[b], vi.uniforms[b], vi.temperature, out[b],
                              acc[b], pd[b])
        checked += 1
    assert checked >= B - 1


def test_max_drafts_per_sequence(gpu):
    """K = 63 drafts per sequence (the limit), rows gathered, mixed temperatures."""
    rng = np.random.default_rng(63)
    B, K, V = 2, 63, 1000
    z = (2.0 * rng.standard_normal((B * K + 5, V))).astype(np.float32)
    rows = rng.permutation(B * K + 5)[:B * K].astype(np.int32).reshape(B, K)
    u = rng.random((B, K), dtype=np.float32)
    temps = np.array([0.0, 0.8], np.float32)
    _parity(gpu, z, "f32", u, 1.0, B, K, row_index=rows, temps=temps)


@pytest.mark.parametrize("V", [8, 2056, 4104, 151936, 155648, 155656])
def test_row_resident_rows(gpu, V):
    """bf16 rows with V a multiple of 8 and q written are held in registers
    when V <= 155648 (a row of up to 76 quads per thread of a 512-thread
    workgroup), else streamed twice.  Both sides of that limit, rows whose
    last quads fill only part of the workgroup (2056, 4104), one-octet rows,
    -inf logits, gathered rows, per-sequence temperatures with greedy rows,
    an invalid row index and the q-less variant; q and the descriptor the
    verify recomputes q from must agree element for element."""
    rng = np.random.default_rng(V + 1)
    B, K = 3, 3
    n = B * K + 2
    z = (3.0 * rng.standard_normal((n, V))).astype(np.float32)
    z[:, :min(V, 16)] += 5.0
    if V > 8:
        z[:, rng.integers(0, V, size=5)] = -np.inf
    logits = synth.f32_to_bf16_bits(z)
    rows = rng.permutation(n)[:B * K].astype(np.int32).reshape(B, K)
    temps = np.array([0.7, 0.0, 1.3], np.float32)
    u = rng.random((B, K), dtype=np.float32)
    tok, q = _parity(gpu, logits, "bf16", u, 1.0, B, K, row_index=rows, temps=temps)
    tok2, _ = _parity(gpu, logits, "bf16", u, 1.0, B, K, row_index=rows, temps=temps,
                      want_q=False)
    assert np.array_equal(tok, tok2)
    # the row descriptors reproduce q exactly as written
    t3, q3, desc = gpu.spec_draft_sample(dev(logits), K, 1.0, uniforms=dev(u),
                                         row_index=dev(rows), temperatures=dev(temps),
                                         want_row_desc=True)
    torch.cuda.synchronize()
    assert np.array_equal(t3.cpu().numpy(), tok)
    assert np.array_equal(q3.cpu().numpy().view(np.int32), q.view(np.int32))
    d = desc.cpu().numpy()                       # [B, K, 4]: c, Mc, 1/S (fp32 bits), token
    zb = logits.astype(np.uint32) << np.uint32(16)
    for b in (0, 2):
        for k in range(K):
            c, mc, inv_s = d[b, k, :3].view(np.float32)
            zr = zb[rows[b, k]].view(np.float32)
            x = np.exp2(np.float64(np.float32(np.float64(zr) * c - mc)))
            assert np.allclose(q[b, k], x * inv_s, rtol=2e-6, atol=1e-37)
    # an invalid row gives token -1 and q = 0; the other rows are unaffected
    bad = rows.copy()
    bad[0, 1] = n
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    t4, q4 = gpu.spec_draft_sample(dev(logits), K, 1.0, uniforms=dev(u), row_index=dev(bad),
                                   temperatures=dev(temps), device_error=err)
    torch.cuda.synchronize()
    t4, q4 = t4.cpu().numpy(), q4.cpu().numpy()
    assert int(err.item()) == gpu.DEVERR_ROW_INDEX
    assert t4[0, 1] == -1 and not q4[0, 1].any()
    keep = np.ones((B, K), bool)
    keep[0, 1] = False
    assert np.array_equal(t4[keep], tok[keep])
    assert np.array_equal(q4[keep].view(np.int32), q[keep].view(np.int32))
