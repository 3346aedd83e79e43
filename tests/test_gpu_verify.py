"""GPU parity: spec_verify_greedy / spec_verify_sample against the oracle.

Token ids and accept lengths are compared exactly; decisions that lie within
1e-6 of their threshold may take either branch (the oracle enumerates the
acceptable outcomes, see oracle.sample_outcomes); p_k(d_k) within 1e-5
relative.  The tiny (B=1, V=32), mid-size (B=8, V=32000) and large-vocabulary
(B=64, V=201088) workloads at full size, ragged and degenerate shapes,
ties, -inf logits, zero draft probabilities, the residual fallback, final
uniforms at 0 and just below 1, invalid draft tokens, determinism, and
chi-square tests of the GPU's own outputs.
"""
import numpy as np
import pytest
import torch
from scipy import stats
from scipy.special import softmax

import oracle
import synth
from tests.gpu_util import DEV, check_sample_sequence, dev

pytestmark = pytest.mark.gpu


def _greedy_parity(sv, logits, dtype, d):
    out, acc = sv.spec_verify_greedy(dev(logits), dev(d))
    torch.cuda.synchronize()
    want_out, want_acc = oracle.verify_greedy(logits, dtype, d)
    assert np.array_equal(acc.cpu().numpy(), want_acc)
    assert np.array_equal(out.cpu().numpy(), want_out)


def _sample_parity(sv, logits, dtype, q, d, u, T, max_flag_frac=0.01, max_mismatch=None):
    out, acc, pd = sv.spec_verify_sample(dev(logits), dev(q), dev(d), dev(u), T,
                                         want_draft_target_prob=True)
    torch.cuda.synchronize()
    out, acc, pd = out.cpu().numpy(), acc.cpu().numpy(), pd.cpu().numpy()
    B = logits.shape[0]
    mism = flags = 0
    for b in range(B):
        z64 = oracle.decode_logits(logits[b], dtype)
        same, f = check_sample_sequence(z64, q[b], d[b], u[b], T, out[b], acc[b], pd[b])
        mism += not same
        flags += f
    assert mism <= flags          # every departure from the canonical outcome is a near tie
    assert flags <= max(2, max_flag_frac * B * (d.shape[1] + 1))
    if max_mismatch is not None:
        assert mism <= max_mismatch
    return out, acc


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_greedy_workloads(gpu, cfg):
    vi = synth.make_verify_inputs(synth.verify_config(cfg))
    _greedy_parity(gpu, vi.logits, vi.spec.dtype, vi.draft_tokens)


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_sample_workloads(gpu, cfg):
    vi = synth.make_verify_inputs(synth.verify_config(cfg))
    _sample_parity(gpu, vi.logits, vi.spec.dtype, vi.draft_probs, vi.draft_tokens, vi.uniforms,
                   vi.temperature)


def _random_case(rng, B, K, V, dtype, T=1.0, tie_heavy=False):
    z = (2.5 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    if tie_heavy:
        z = np.round(z * 2) / 2                      # many exact ties
    if dtype == "bf16":
        logits = synth.f32_to_bf16_bits(z)
        z = synth.bf16_bits_to_f32(logits)
    else:
        logits = z
    q = softmax(z[:, :K].astype(np.float64) / T + rng.standard_normal((B, K, V)), axis=2)
    q32 = q.astype(np.float32)
    d = np.zeros((B, K), np.int32)
    for b in range(B):
        for k in range(K):
            d[b, k] = rng.choice(V, p=q[b, k])
    u = rng.random((B, K + 1), dtype=np.float32)
    return logits, q32, d, u


RAGGED = [  # (dtype, B, K, V)
    ("f32", 3, 2, 1), ("bf16", 2, 1, 7), ("f32", 5, 4, 33), ("bf16", 4, 3, 1001),
    ("f32", 2, 5, 4099), ("bf16", 3, 63, 600), ("f32", 2, 0, 100), ("bf16", 300, 3, 64),
    ("bf16", 2, 2, 24576), ("f32", 1, 1, 65544), ("bf16", 9, 7, 513),
]


@pytest.mark.parametrize("dtype,B,K,V", RAGGED)
def test_ragged_shapes(gpu, dtype, B, K, V):
    rng = np.random.default_rng(B * 1000 + K * 10 + V)
    logits, q, d, u = _random_case(rng, B, K, V, dtype, T=0.8, tie_heavy=True)
    _greedy_parity(gpu, logits, dtype, d)
    _sample_parity(gpu, logits, dtype, q, d, u, 0.8)


@pytest.mark.parametrize("dtype,V", [("f32", 5000), ("bf16", 30000)])
def test_extreme_final_uniforms(gpu, dtype, V):
    """The final draw at u = 0 (the first token with positive mass) and at the
    largest fp32 below 1 (u*S at or past the rounded total: the last token
    with positive mass), for residual draws and bonus draws."""
    rng = np.random.default_rng(V + 11)
    B, K = 16, 3
    logits, q, d, u = _random_case(rng, B, K, V, dtype, T=0.9)
    top = np.nextafter(np.float32(1), np.float32(0))
    u[:, K] = np.where(np.arange(B) % 2 == 0, np.float32(0), top)
    u[:8, :K] = 0.0            # accept every draft with p > 0: bonus draws from p_K
    u[8:, 0] = top             # reject draft 0 unless p/q >= 1: residual draws from row 0
    # u*S lies within 1e-6 of the CDF's first or last boundary by construction,
    # so every final draw is a flagged near tie; the GPU's token must still be
    # one the oracle allows, and the oracle's own choice in all but a few
    _sample_parity(gpu, logits, dtype, q, d, u, 0.9, max_flag_frac=1.0, max_mismatch=2)


def test_max_vocab(gpu):
    rng = np.random.default_rng(3)
    logits, q, d, u = _random_case(rng, 2, 2, 1 << 19, "bf16", T=1.3)
    _greedy_parity(gpu, logits, "bf16", d)
    _sample_parity(gpu, logits, "bf16", q, d, u, 1.3)


@pytest.mark.parametrize("V", [8992, 16392, 16387])
def test_fp32_rows_wave_blocks(gpu, V):
    """fp32 logits on rows long enough for the row kernel's wave-block loop
    (B(K+1) = 2048 rows, one workgroup per row; each lane holds two quads of
    a wave's 512-element block): the lowest-index argmax of every row on
    tie-heavy logits, and sampling against the oracle.  V = 8992 leaves a
    partial step for the per-octet loop, V = 16387 (not a multiple of 8) takes
    the per-element loads."""
    rng = np.random.default_rng(V)
    B, K = 256, 7
    logits, q, d, u = _random_case(rng, B, K, V, "f32", T=0.9, tie_heavy=True)
    _greedy_parity(gpu, logits, "f32", d)
    _sample_parity(gpu, logits, "f32", q, d, u, 0.9)


def test_fp32_split_rows_wave_blocks(gpu):
    """fp32 rows split over 16 workgroups (B(K+1) = 4 rows) whose slices of
    ~2050 octets start at octets that are not multiples of 64: the wave-block
    loop on unaligned slice starts, then the per-octet tail."""
    rng = np.random.default_rng(262440)
    B, K, V = 2, 1, 262440
    logits, q, d, u = _random_case(rng, B, K, V, "f32", T=1.1, tie_heavy=True)
    _greedy_parity(gpu, logits, "f32", d)
    _sample_parity(gpu, logits, "f32", q, d, u, 1.1)


def test_greedy_lowest_index_across_splits(gpu):
    B, K, V = 2, 1, 32000               # several workgroups share a row
    z = np.full((B, K + 1, V), -5.0, np.float32)
    z[0, 0, [31999, 5000, 20000]] = 9.0
    z[0, 1, [7, 6]] = 1.0
    z[1, 0, 17] = -0.0                  # -0 and +0 tie at the top: index 3 wins
    z[1, 0, 3] = 0.0
    z[1, 1, 100] = -0.0
    z[1, 1, 200] = 0.0
    d = np.array([[5000], [3]], np.int32)
    out, acc = gpu.spec_verify_greedy(dev(z), dev(d))
    torch.cuda.synchronize()
    assert acc.cpu().tolist() == [1, 1]
    assert out.cpu().tolist() == [[5000, 6], [3, 100]]
    _greedy_parity(gpu, z, "f32", d)
    zb = synth.f32_to_bf16_bits(z)
    _greedy_parity(gpu, zb, "bf16", d)


def test_neg_inf_logits(gpu):
    rng = np.random.default_rng(4)
    logits, q, d, u = _random_case(rng, 6, 3, 300, "f32")
    logits[:, :, ::3] = -np.inf                       # a third of the vocabulary is impossible
    logits[0, 1, :] = -np.inf                         # a whole row of -inf (greedy only)
    _greedy_parity(gpu, logits, "f32", d)
    logits[0, 1, :150] = 1.0
    logits[0, 1, ::3] = -np.inf
    q = q.copy()
    q[:, :, ::3] = 0.0
    d[:, :] = 1
    _sample_parity(gpu, logits, "f32", q, d, u, 1.0)


def test_zero_draft_probability(gpu):
    # q_k(d) = 0: kept when p_k(d) > 0, rejected when p_k(d) = 0
    B, K, V = 4, 2, 50
    rng = np.random.default_rng(5)
    logits, q, d, u = _random_case(rng, B, K, V, "f32")
    for b in range(B):
        for k in range(K):
            q[b, k, d[b, k]] = 0.0
    logits[1, 0, d[1, 0]] = -np.inf
    out, acc = _sample_parity(gpu, logits, "f32", q, d, u, 1.0)
    assert acc[1] == 0
    assert acc[0] >= 1 and acc[2] >= 1 and acc[3] >= 1


@pytest.mark.parametrize("V", [40, 5000, 20000, 40000])
def test_residual_fallback_to_p(gpu, V):
    # q = 2p: every test accepts with probability 1/2 and the residual is zero.
    # V = 40, 5000, 20000: one draw workgroup per sequence with its tiles in
    # registers (1, 3 and 10 CDF tiles; the fallback to p loads the chosen
    # tile again); V = 40000: several draw workgroups per sequence and the
    # locate kernel.
    B, K = 64, 3
    rng = np.random.default_rng(6)
    z = (2 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    p = softmax(z.astype(np.float64), axis=2)
    q = (2 * p[:, :K]).astype(np.float32)
    d = np.array([[rng.choice(V, p=p[b, k]) for k in range(K)] for b in range(B)], np.int32)
    u = rng.random((B, K + 1), dtype=np.float32)
    out, acc = _sample_parity(gpu, z, "f32", q, d, u, 1.0)
    assert (acc < K).any()


def test_q_equals_p_accepts_all(gpu):
    B, K, V = 32, 4, 64
    z = np.zeros((B, K + 1, V), np.float32)           # uniform rows: p = 1/64 exactly
    q = np.full((B, K, V), 1.0 / 64, np.float32)
    rng = np.random.default_rng(7)
    d = rng.integers(0, V, size=(B, K)).astype(np.int32)
    u = rng.random((B, K + 1), dtype=np.float32)
    out, acc = _sample_parity(gpu, z, "f32", q, d, u, 1.0)
    assert np.all(acc == K)


def test_invalid_draft_tokens(gpu):
    rng = np.random.default_rng(8)
    logits, q, d, u = _random_case(rng, 3, 3, 64, "f32")
    d[0, 0] = 64
    d[1, 1] = -5
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, acc, pd = gpu.spec_verify_sample(dev(logits), dev(q), dev(d), dev(u), 1.0,
                                          want_draft_target_prob=True, device_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) & gpu.DEVERR_DRAFT_TOKEN
    acc = acc.cpu().numpy()
    assert acc[0] == 0 and acc[1] <= 1
    assert pd[0, 0].item() == 0.0 and pd[1, 1].item() == 0.0
    err.zero_()
    out, acc = gpu.spec_verify_greedy(dev(logits), dev(d), device_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) & gpu.DEVERR_DRAFT_TOKEN
    assert acc[0].item() == 0
    assert 0 <= out[0, 0].item() < 64


def test_empty_batch(gpu):
    z = torch.zeros((0, 4, 32), device=DEV)
    d = torch.zeros((0, 3), dtype=torch.int32, device=DEV)
    out, acc = gpu.spec_verify_greedy(z, d)
    assert out.shape == (0, 4) and acc.shape == (0,)


@pytest.mark.parametrize("whole", [False, True])
def test_determinism_poison_and_clean_workspace(gpu, whole):
    """Two runs on poisoned outputs give identical bytes and leave the
    workspace all zero: with several draw workgroups per sequence (and the
    locate kernel), and with one draw workgroup per sequence that keeps its
    row's tiles in registers (V = 1000), where the draw workgroup clears the
    row partials."""
    if whole:
        rng = np.random.default_rng(12)
        logits, q, d, u = _random_case(rng, 16, 7, 1000, "f32", T=0.7)
        args, V, T = [dev(logits), dev(q), dev(d), dev(u)], 1000, 0.7
    else:
        vi = synth.make_verify_inputs(synth.verify_config(4), seqs=range(16))
        args = [dev(vi.logits), dev(vi.draft_probs), dev(vi.draft_tokens), dev(vi.uniforms)]
        V, T = 201088, vi.temperature
    ws = torch.zeros(gpu.spec_verify_workspace_bytes(16, 7, V), dtype=torch.uint8, device=DEV)
    res = []
    for poison in (0x7F7F7F7F, -0x10101011):
        out = torch.full((16, 8), poison, dtype=torch.int32, device=DEV)
        acc = torch.full((16,), poison, dtype=torch.int32, device=DEV)
        pd = torch.full((16, 7), float("nan"), device=DEV)
        gpu.spec_verify_sample(*args, T, out_tokens=out, out_num_accepted=acc,
                               out_draft_target_prob=pd, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero().item()) == 0        # tickets reset by the kernel
        res.append((out.cpu().numpy(), acc.cpu().numpy(), pd.cpu().numpy()))
    for x, y in zip(res[0], res[1]):
        assert x.tobytes() == y.tobytes()
    assert np.all(np.isfinite(res[0][2]))


@pytest.mark.parametrize("V,N", [(4, 200_000), (8, 200_000), (32, 100_000)])
def test_chi_square_on_gpu_outputs(gpu, V, N):
    """The GPU's emitted tokens follow the target (same tests as the oracle's)."""
    K, T = 3, 1.0
    rng = np.random.default_rng(100 + V)
    z = (2.0 * rng.standard_normal((K + 1, V))).astype(np.float32)
    q = softmax(z[:K].astype(np.float64) + rng.standard_normal((K, V)), axis=1).astype(np.float32)
    qn = q.astype(np.float64) / q.astype(np.float64).sum(axis=1, keepdims=True)
    d = np.stack([rng.choice(V, size=N, p=qn[k]) for k in range(K)], axis=1).astype(np.int32)
    u = rng.random((N, K + 1), dtype=np.float32)
    zt = dev(z).unsqueeze(0).expand(N, K + 1, V).contiguous()
    qt = dev(q).unsqueeze(0).expand(N, K, V).contiguous()
    out, acc, _ = gpu.spec_verify_sample(zt, qt, dev(d), dev(u), T)
    torch.cuda.synchronize()
    out, acc = out.cpu().numpy(), acc.cpu().numpy()
    p = [softmax(z[k].astype(np.float64) / T) for k in range(K + 1)]

    def chi2(sample, probs):
        counts = np.bincount(sample, minlength=V)
        keep = probs * len(sample) >= 5
        assert counts[probs == 0].sum() == 0
        obs = np.concatenate([counts[keep], [counts[~keep].sum()]])
        exp = np.concatenate([probs[keep], [probs[~keep].sum()]]) * len(sample)
        if exp[-1] == 0:
            obs, exp = obs[:-1], exp[:-1]
        return stats.chisquare(obs, exp).pvalue

    assert chi2(out[:, 0], p[0]) > 1e-4
    assert chi2(out[acc >= 1, 1], p[1]) > 1e-4
    beta = [np.minimum(p[k], q[k].astype(np.float64)).sum() for k in range(K)]
    assert stats.binomtest(int((acc >= 1).sum()), N, beta[0]).pvalue > 1e-4
    want = sum(np.prod(beta[:k]) for k in range(1, K + 1))
    assert abs(acc.mean() - want) < 4.5 * acc.std() / np.sqrt(N)


def test_workspace_reuse_across_shapes(gpu):
    """One workspace shared by calls of different (B, K, V): every call leaves
    it all zeros, so a later call's tickets never meet stale partials."""
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    rng = np.random.default_rng(12)
    for dtype, B, K, V in [("bf16", 64, 7, 20000), ("bf16", 300, 3, 64), ("f32", 9, 5, 3000),
                           ("bf16", 500, 1, 640)]:
        logits, q, d, u = _random_case(rng, B, K, V, dtype)
        out, acc = gpu.spec_verify_greedy(dev(logits), dev(d), workspace=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero().item()) == 0
        want_out, want_acc = oracle.verify_greedy(logits, dtype, d)
        assert np.array_equal(acc.cpu().numpy(), want_acc)
        assert np.array_equal(out.cpu().numpy(), want_out)
        out, acc, _ = gpu.spec_verify_sample(dev(logits), dev(q), dev(d), dev(u), 1.0, workspace=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero().item()) == 0
        for b in range(0, B, max(1, B // 16)):
            check_sample_sequence(oracle.decode_logits(logits[b], dtype), q[b], d[b], u[b], 1.0,
                                  out[b].cpu().numpy(), acc[b].item())


@pytest.mark.parametrize("dtype,B,V", [("bf16", 256, 40000), ("f32", 256, 40001),
                                        ("bf16", 300, 40000), ("f32", 260, 40001),
                                        ("bf16", 700, 40000)])
def test_one_wide_draw_workgroup_per_sequence(gpu, dtype, B, V):
    """Mid-size batches (256 <= B < 854) with rows of more than 16 CDF
    tiles: one draw workgroup per sequence searches the token itself (no
    locate kernel), 1024 threads wide at B = 256, 512 at B = 300 and 260, 256
    at B = 700; parity with the oracle, run-to-run identical outputs and a
    workspace left all zero.  V = 40001 takes the per-element loads."""
    rng = np.random.default_rng(B + V)
    K = 3
    logits, q, d, u = _random_case(rng, B, K, V, dtype, T=0.9)
    # with ~40000 CDF cells of ~2.5e-5 each, u*S lands within the 1e-6 band
    # of a cell boundary on ~8% of the draws (flags of the inputs, not of the
    # GPU; every departure from the canonical outcome must still be one)
    _sample_parity(gpu, logits, dtype, q, d, u, 0.9, max_flag_frac=0.1)
    ws = torch.zeros(gpu.spec_verify_workspace_bytes(B, K, V), dtype=torch.uint8, device=DEV)
    out, acc, _ = gpu.spec_verify_sample(dev(logits), dev(q), dev(d), dev(u), 0.9, workspace=ws)
    torch.cuda.synchronize()
    assert int(ws.count_nonzero().item()) == 0
    out2, acc2, _ = gpu.spec_verify_sample(dev(logits), dev(q), dev(d), dev(u), 0.9, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(acc, acc2)


def test_max_batch(gpu):
    """B = SV_MAX_B sequences (K = 1, V = 16, fp32): every sequence against
    the greedy definition (numpy lowest-index argmax) and, sampled, against
    well-formedness and the support of the drawn token; a seeded sample of
    sequences against the oracle."""
    B, K, V, T = gpu.MAX_B, 1, 16, 1.0
    rng = np.random.default_rng(20)
    z = (2 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    q = softmax(z[:, :K].astype(np.float64) + rng.standard_normal((B, K, V)), axis=2)
    cdf = np.cumsum(q[:, 0], axis=1)
    d = np.minimum((cdf < rng.random((B, 1))).sum(axis=1), V - 1).astype(np.int32)[:, None]
    q32 = q.astype(np.float32)
    u = rng.random((B, K + 1), dtype=np.float32)
    out, acc = gpu.spec_verify_greedy(dev(z), dev(d))
    torch.cuda.synchronize()
    out, acc = out.cpu().numpy(), acc.cpu().numpy()
    g = np.argmax(z, axis=2)
    want_a = (d[:, 0] == g[:, 0]).astype(np.int32)
    assert np.array_equal(acc, want_a)
    rows = np.arange(B)
    assert np.array_equal(out[rows, acc], g[rows, acc])
    assert np.all(out[acc == 0, 1] == -1)
    out, acc, _ = gpu.spec_verify_sample(dev(z), dev(q32), dev(d), dev(u), T)
    torch.cuda.synchronize()
    out, acc = out.cpu().numpy(), acc.cpu().numpy()
    assert np.all((acc == 0) | (acc == 1))
    assert np.array_equal(out[acc == 1, 0], d[acc == 1, 0])
    c = out[rows, acc]
    assert np.all((c >= 0) & (c < V)) and np.all(out[acc == 0, 1] == -1)
    p = softmax(z.astype(np.float64) / T, axis=2)
    pc = p[rows, acc, c]
    qc = np.where(acc == 0, q32[rows, 0, c].astype(np.float64), 0.0)
    assert np.all(pc > qc * (1 - 1e-5))              # the residual's support (p for the bonus)
    for b in rng.choice(B, 64, replace=False):
        check_sample_sequence(z[b].astype(np.float64), q32[b], d[b], u[b], T, out[b], acc[b])


TILES_IN_REGISTERS = [  # (dtype, B, K, V, mode): rows of at most 16 CDF tiles
    ("f32", 8, 5, 32000, "dense"), ("bf16", 40, 7, 32768, "dense"), ("bf16", 17, 3, 2048, "dense"),
    ("f32", 33, 4, 8192, "dense"), ("bf16", 5, 2, 8200, "dense"), ("f32", 6, 3, 16383, "dense"),
    ("bf16", 300, 3, 12000, "dense"), ("bf16", 24, 7, 30000, "lq"), ("f32", 12, 4, 12000, "lq"),
    ("f32", 9, 3, 16385, "lq"), ("bf16", 20, 5, 20000, "mixed"), ("f32", 14, 3, 6001, "mixed"),
]


@pytest.mark.parametrize("dtype,B,K,V,mode", TILES_IN_REGISTERS)
def test_tiles_in_registers(gpu, dtype, B, K, V, mode):
    """Rows of at most 16 CDF tiles (8 when the rows are not vectorised or are
    fp32 rows with q from the drafter logits): one draw workgroup per
    sequence keeps its tiles in registers and draws the token without loading
    them again.  Every sequence against the oracle, final uniforms at 0 and
    just below 1 on some sequences, run-to-run identical outputs, and a
    workspace left all zero; q from the drafter logits equals the dense-q
    verify bit for bit, and mixed batches match the oracle per sequence."""
    rng = np.random.default_rng(B * 131 + V + K)
    logits, q, d, u = _random_case(rng, B, K, V, dtype, T=0.8)
    u[::5, K] = 0.0
    u[1::5, K] = np.nextafter(np.float32(1.0), np.float32(0.0))
    ws = torch.zeros(gpu.spec_verify_workspace_bytes(B, K, V), dtype=torch.uint8, device=DEV)
    if mode == "dense":
        outs = []
        for _ in range(2):
            out, acc, pd = gpu.spec_verify_sample(dev(logits), dev(q), dev(d), dev(u), 0.8,
                                                  want_draft_target_prob=True, workspace=ws)
            torch.cuda.synchronize()
            assert int(ws.count_nonzero().item()) == 0
            outs.append((out.cpu().numpy(), acc.cpu().numpy(), pd.cpu().numpy()))
        assert all(np.array_equal(x, y) for x, y in zip(*outs))
        out, acc, pd = outs[0]
        for b in range(B):
            check_sample_sequence(oracle.decode_logits(logits[b], dtype), q[b], d[b], u[b], 0.8,
                                  out[b], acc[b], pd[b])
    elif mode == "lq":
        from tests.test_gpu_lq import _chain, _same
        zd = (2.5 * rng.standard_normal((B * K, V))).astype(np.float32)
        if dtype == "bf16":
            zd = synth.f32_to_bf16_bits(zd)
        ud = rng.random((B, K), dtype=np.float32)
        _, _, _, dense, lq = _chain(gpu, dev(logits), dev(zd), K, 0.8, 0.9, dev(ud), dev(u))
        _same(dense, lq)
    else:
        from types import SimpleNamespace
        from tests.test_gpu_mixed import _mixed_parity
        vi = SimpleNamespace(logits=logits, draft_probs=q, draft_tokens=d, uniforms=u,
                             spec=SimpleNamespace(B=B, dtype=dtype))
        temps = np.where(np.arange(B) % 3 == 0, 0.0, 0.6 + 0.05 * (np.arange(B) % 7)).astype(np.float32)
        _mixed_parity(gpu, vi, temps)
