"""GPU: the early-exit verify forms (spec_verify_greedy_early_exit,
spec_verify_sample_early_exit, spec_verify_mixed_early_exit).

Each computes a sequence's row statistics only up to its first rejection,
one launch per draft position.  Its tokens, accept counts and device flags
must equal the full call's bit for bit, p_k(d_k) must equal the full call's
for k <= a and be 0 past it, and the workspace must be left all zero.
Covered: the tiny, mid and large-vocabulary workloads, a 48-sequence slice
of the 1024-sequence batch, 300 sequences (one draw workgroup per
sequence), the ragged shapes of the verify tests (K = 0 and 63, V = 1, V
not a multiple of 8), every draft accepted, every sequence rejected at its
first draft, invalid draft tokens, mixed batches with greedy sequences,
SV_MAX_B sequences, the drafter-logit forms; and the oracle directly on the
mid workload.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import DEV, check_sample_sequence, dev
from tests.test_gpu_verify import RAGGED, _random_case

pytestmark = pytest.mark.gpu


def _ws(sv, B, K, V):
    return torch.zeros(max(1, sv.spec_verify_workspace_bytes(B, K, V)), dtype=torch.uint8,
                       device=DEV)


def _prefix_equal(full, ee):
    """Tokens and counts equal; p_k(d_k) equal for k <= a and 0 past it."""
    out, acc, pd = full
    eo, ea, ep = ee
    assert torch.equal(out, eo) and torch.equal(acc, ea)
    K = pd.shape[1]
    keep = torch.arange(K, device=DEV)[None, :] <= acc.long()[:, None]
    want = torch.where(keep, pd, torch.zeros_like(pd))
    assert torch.equal(want.view(torch.int32), ep.view(torch.int32))


def _compare(sv, logits, dtype, q, d, u, T, temps=None):
    """Greedy, sampled and (with temps) mixed calls, full and early exit."""
    B, K1, V = logits.shape
    K = K1 - 1
    z, qd, dd, ud = dev(logits), dev(q), dev(d), dev(u)
    errs = [torch.zeros(1, dtype=torch.int32, device=DEV) for _ in range(6)]
    ws = [_ws(sv, B, K, V) for _ in range(6)]
    g_full = sv.spec_verify_greedy(z, dd, workspace=ws[0], device_error=errs[0])
    g_ee = sv.spec_verify_greedy_early_exit(z, dd, workspace=ws[1], device_error=errs[1])
    s_full = sv.spec_verify_sample(z, qd, dd, ud, T, want_draft_target_prob=True,
                                   workspace=ws[2], device_error=errs[2])
    s_ee = sv.spec_verify_sample_early_exit(z, qd, dd, ud, T, want_draft_target_prob=True,
                                            workspace=ws[3], device_error=errs[3])
    if temps is not None:
        tt = dev(temps)
        m_full = sv.spec_verify_mixed(z, qd, dd, ud, tt, want_draft_target_prob=True,
                                      workspace=ws[4], device_error=errs[4])
        m_ee = sv.spec_verify_mixed_early_exit(z, qd, dd, ud, tt, want_draft_target_prob=True,
                                               workspace=ws[5], device_error=errs[5])
    torch.cuda.synchronize()
    assert torch.equal(g_full[0], g_ee[0]) and torch.equal(g_full[1], g_ee[1])
    _prefix_equal(s_full, s_ee)
    if temps is not None:
        _prefix_equal(m_full, m_ee)
    n = 6 if temps is not None else 4
    for i in range(0, n, 2):
        assert int(errs[i].item()) == int(errs[i + 1].item()), i
    for w in ws[:n]:
        assert int(w.count_nonzero().item()) == 0
    return g_ee, s_ee


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_workloads(gpu, cfg):
    vi = synth.make_verify_inputs(synth.verify_config(cfg))
    temps = synth.make_temperatures(vi.spec.B, 40 + cfg)
    _compare(gpu, vi.logits, vi.spec.dtype, vi.draft_probs, vi.draft_tokens, vi.uniforms,
             vi.temperature, temps)


def test_large_batch_slice(gpu):
    vi = synth.make_verify_inputs(synth.verify_config(5), seqs=range(48))
    _, (out, acc, _) = _compare(gpu, vi.logits, vi.spec.dtype, vi.draft_probs, vi.draft_tokens,
                                vi.uniforms, vi.temperature, synth.make_temperatures(48, 45))
    assert 0 < int(acc.sum().item()) < 48 * vi.spec.K


def test_one_draw_workgroup_per_sequence(gpu):
    rng = np.random.default_rng(301)
    logits, q, d, u = _random_case(rng, 300, 4, 40000, "bf16", T=0.8)
    _compare(gpu, logits, "bf16", q, d, u, 0.8, synth.make_temperatures(300, 46))


@pytest.mark.parametrize("dtype,B,K,V", RAGGED)
def test_ragged_shapes(gpu, dtype, B, K, V):
    rng = np.random.default_rng(B * 1000 + K * 10 + V + 5)
    logits, q, d, u = _random_case(rng, B, K, V, dtype, T=0.8, tie_heavy=True)
    _compare(gpu, logits, dtype, q, d, u, 0.8, synth.make_temperatures(B, 47))


@pytest.mark.parametrize("dtype,B,K,V", [("bf16", 640, 7, 5003), ("f32", 520, 15, 2048),
                                         ("bf16", 130, 5, 3001), ("bf16", 130, 63, 300),
                                         ("f32", 512, 31, 264)])
def test_gate_kernels(gpu, dtype, B, K, V):
    """Batches large enough for the gate kernels and listed ranges (greedy
    from 128 sequences, sampled and mixed from 512), with the greedy form's
    finer row splits, on tie-heavy rows: identical to the full calls, and the
    workspace (counters and list included) left zero."""
    rng = np.random.default_rng(B * 7 + K + V)
    logits, q, d, u = _random_case(rng, B, K, V, dtype, T=0.8, tie_heavy=True)
    _compare(gpu, logits, dtype, q, d, u, 0.8, synth.make_temperatures(B, 50))


def test_all_accepted_and_first_rejected(gpu):
    rng = np.random.default_rng(302)
    B, K, V = 12, 7, 5000
    logits, q, d, u = _random_case(rng, B, K, V, "f32", T=1.0)
    z = logits[:, :K]
    top = np.argmax(z, axis=2).astype(np.int32)          # unique maxima for N(0, 2.5^2) logits
    # every draft is the row's argmax with q = one-hot and u = 0: accepted by
    # the greedy rule and by rejection sampling (u < p / q since p > 0)
    q1 = np.zeros_like(q)
    np.put_along_axis(q1, top[:, :, None], 1.0, axis=2)
    u0 = u.copy()
    u0[:, :K] = 0.0
    (go, ga), (so, sa, _) = _compare(gpu, logits, "f32", q1, top, u0, 1.0)
    assert ga.cpu().tolist() == [K] * B and sa.cpu().tolist() == [K] * B
    # the first draft never the argmax, with q = one-hot on it and u just
    # below 1: rejected at once by both rules (p / q < 1 there)
    d1 = top.copy()
    d1[:, 0] = (top[:, 0] + 1) % V
    q2 = q1.copy()
    q2[:, 0] = 0.0
    q2[np.arange(B), 0, d1[:, 0]] = 1.0
    u1 = u0.copy()
    u1[:, 0] = np.float32(1.0) - np.float32(2.0 ** -24)
    (go, ga), (so, sa, _) = _compare(gpu, logits, "f32", q2, d1, u1, 1.0)
    assert ga.cpu().tolist() == [0] * B and sa.cpu().tolist() == [0] * B


def test_invalid_draft_tokens(gpu):
    rng = np.random.default_rng(303)
    logits, q, d, u = _random_case(rng, 6, 5, 3000, "bf16", T=0.9)
    d[1, 0] = -3                       # rejected at the first draft, flagged
    d[2, 3] = 3000                     # past the vocabulary
    d[4, 4] = 1 << 30
    _compare(gpu, logits, "bf16", q, d, u, 0.9, synth.make_temperatures(6, 48))


def test_sample_matches_oracle(gpu):
    """The sampled early-exit call against the oracle on the mid workload:
    outcomes within the 1e-6 near-tie rule, p_k(d_k) for k <= a."""
    vi = synth.make_verify_inputs(synth.verify_config(2))
    out, acc, pd = gpu.spec_verify_sample_early_exit(dev(vi.logits), dev(vi.draft_probs),
                                                     dev(vi.draft_tokens), dev(vi.uniforms),
                                                     vi.temperature, want_draft_target_prob=True)
    torch.cuda.synchronize()
    out, acc, pd = out.cpu().numpy(), acc.cpu().numpy(), pd.cpu().numpy()
    for b in range(vi.spec.B):
        z64 = oracle.decode_logits(vi.logits[b], vi.spec.dtype)
        check_sample_sequence(z64, vi.draft_probs[b], vi.draft_tokens[b], vi.uniforms[b],
                              vi.temperature, out[b], acc[b])
        a = int(acc[b])
        for k in range(vi.spec.K):
            want = oracle.target_distribution(z64[k], vi.temperature)[int(vi.draft_tokens[b, k])]
            if k <= a:
                assert np.isclose(pd[b, k], want, rtol=1e-5, atol=1e-30), (b, k)
            else:
                assert pd[b, k] == 0.0


@pytest.mark.parametrize("dtype,B,K,V", [("bf16", 40, 7, 151936), ("f32", 9, 5, 4099),
                                         ("bf16", 300, 3, 40000), ("bf16", 520, 3, 3000)])
def test_drafter_logit_forms(gpu, dtype, B, K, V):
    """spec_verify_sample_lq_early_exit and spec_verify_mixed_lq_early_exit
    against the full drafter-logit calls on the same drafting (drafter rows
    gathered through a row index, one of them invalid at a sampled sequence's
    first draft: the same flag)."""
    rng = np.random.default_rng(B + K + V)
    z = (3.0 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
    z[:, :, :8] += 6.0
    n = B * K
    zd = np.concatenate([(z[:, :K] + rng.standard_normal((B, K, V)).astype(np.float32))
                         .reshape(n, V), np.zeros((2, V), np.float32)])
    if dtype == "bf16":
        z, zd = synth.f32_to_bf16_bits(z), synth.f32_to_bf16_bits(zd)
    rows = rng.permutation(n).astype(np.int32).reshape(B, K)
    ud = rng.random((B, K), dtype=np.float32)
    uv = rng.random((B, K + 1), dtype=np.float32)
    temps = synth.make_temperatures(B, 49)
    zt, zdt, rt, uvt = dev(z), dev(zd), dev(rows), dev(uv)
    for mixed in (False, True):
        tok, _, desc = gpu.spec_draft_sample(zdt, K, 0.8, uniforms=dev(ud), row_index=rt,
                                             temperatures=dev(temps) if mixed else None,
                                             want_draft_probs=False, want_row_desc=True)
        bad = rows.copy()
        bb = int(np.argmax(temps > 0))                         # a sampled sequence
        bad[bb, 0] = n + 7                                     # no such drafter row
        badt = dev(bad)
        errs = [torch.zeros(1, dtype=torch.int32, device=DEV) for _ in range(2)]
        wss = [_ws(gpu, B, K, V) for _ in range(2)]
        if mixed:
            args = (zt, zdt, desc, tok, uvt, dev(temps))
            full = gpu.spec_verify_mixed_lq(*args, drafter_rows=badt, want_draft_target_prob=True,
                                            workspace=wss[0], device_error=errs[0])
            ee = gpu.spec_verify_mixed_lq_early_exit(*args, drafter_rows=badt,
                                                     want_draft_target_prob=True,
                                                     workspace=wss[1], device_error=errs[1])
        else:
            args = (zt, zdt, desc, tok, uvt, 0.9)
            full = gpu.spec_verify_sample_lq(*args, drafter_rows=badt, want_draft_target_prob=True,
                                             workspace=wss[0], device_error=errs[0])
            ee = gpu.spec_verify_sample_lq_early_exit(*args, drafter_rows=badt,
                                                      want_draft_target_prob=True,
                                                      workspace=wss[1], device_error=errs[1])
        torch.cuda.synchronize()
        _prefix_equal(full, ee)
        assert int(errs[0].item()) == int(errs[1].item()) != 0
        for w in wss:
            assert int(w.count_nonzero().item()) == 0


def test_max_batch(gpu):
    """B = SV_MAX_B sequences (K = 1, V = 16, fp32; K = 3 with V = 8 for the
    ranges [1,2) and [2,4)): the early-exit forms equal the full calls."""
    for K, V in ((1, 16), (3, 8)):
        B = gpu.MAX_B if K == 1 else gpu.MAX_B // 4
        rng = np.random.default_rng(21 + K)
        z = (2 * rng.standard_normal((B, K + 1, V))).astype(np.float32)
        q = np.full((B, K, V), 1.0 / V, np.float32)
        d = rng.integers(0, V, size=(B, K)).astype(np.int32)
        u = rng.random((B, K + 1), dtype=np.float32)
        _compare(gpu, z, "f32", q, d, u, 1.0)


def test_gate_kernels_in_a_captured_graph(gpu):
    """The early-exit calls with gate kernels (B = 520: greedy, sampled and
    mixed) captured in one torch graph and replayed on new uniforms and
    drafts, with the library's eager calls between replays: every replay
    equals the eager full calls on its inputs (p_k(d_k) up to the first
    rejection), and leaves the workspaces zero."""
    B, K, V = 520, 5, 3001
    rng = np.random.default_rng(77)
    logits, q, d, u = _random_case(rng, B, K, V, "bf16", T=0.8)
    temps = dev(synth.make_temperatures(B, 51))
    z, qd, dd, ud = dev(logits), dev(q), dev(d), dev(u)
    ws = [_ws(gpu, B, K, V) for _ in range(3)]
    outs = [(torch.empty((B, K + 1), dtype=torch.int32, device=DEV),
             torch.empty((B,), dtype=torch.int32, device=DEV),
             torch.empty((B, K), dtype=torch.float32, device=DEV)) for _ in range(3)]

    def calls():
        gpu.spec_verify_greedy_early_exit(z, dd, out_tokens=outs[0][0], out_num_accepted=outs[0][1],
                                          workspace=ws[0])
        gpu.spec_verify_sample_early_exit(z, qd, dd, ud, 0.8, out_tokens=outs[1][0],
                                          out_num_accepted=outs[1][1],
                                          out_draft_target_prob=outs[1][2], workspace=ws[1])
        gpu.spec_verify_mixed_early_exit(z, qd, dd, ud, temps, out_tokens=outs[2][0],
                                         out_num_accepted=outs[2][1],
                                         out_draft_target_prob=outs[2][2], workspace=ws[2])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        d_new = d.copy()
        d_new[:, rep % K] = rng.integers(0, V, size=B)
        dd.copy_(dev(d_new))
        ud.copy_(dev(rng.random((B, K + 1), dtype=np.float32)))
        g.replay()
        torch.cuda.synchronize()
        full = (gpu.spec_verify_greedy(z, dd),
                gpu.spec_verify_sample(z, qd, dd, ud, 0.8, want_draft_target_prob=True),
                gpu.spec_verify_mixed(z, qd, dd, ud, temps, want_draft_target_prob=True))
        torch.cuda.synchronize()
        assert torch.equal(full[0][0], outs[0][0]) and torch.equal(full[0][1], outs[0][1]), rep
        _prefix_equal(full[1], outs[1])
        _prefix_equal(full[2], outs[2])
        for w in ws:
            assert int(w.count_nonzero().item()) == 0, rep
    del g
