"""GPU parity: spec_verify_mixed (a temperature per sequence, 0 = greedy).

Greedy sequences are compared exactly (tokens, accept count, and the 0/1
p_draft of the T -> 0 limit); sampled sequences as in the sampled-verify
tests (decisions within 1e-6 of their threshold may go either way, p_k(d_k)
within 1e-5).  A uniform batch must reproduce spec_verify_greedy or
spec_verify_sample bit for bit; invalid temperatures are flagged and verified
greedily.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import DEV, check_sample_sequence, dev

pytestmark = pytest.mark.gpu


def _mixed_parity(sv, vi, temps):
    out, acc, pd = sv.spec_verify_mixed(dev(vi.logits), dev(vi.draft_probs), dev(vi.draft_tokens),
                                        dev(vi.uniforms), dev(temps), want_draft_target_prob=True)
    torch.cuda.synchronize()
    out, acc, pd = out.cpu().numpy(), acc.cpu().numpy(), pd.cpu().numpy()
    mism = flags = 0
    for b in range(vi.spec.B):
        z64 = oracle.decode_logits(vi.logits[b], vi.spec.dtype)
        if oracle.mixed.is_greedy(temps[b]):
            w_out, w_acc, w_pd = oracle.verify_mixed(vi.logits[b:b + 1], vi.spec.dtype,
                                                     vi.draft_probs[b:b + 1],
                                                     vi.draft_tokens[b:b + 1],
                                                     vi.uniforms[b:b + 1], temps[b:b + 1])
            assert acc[b] == w_acc[0] and np.array_equal(out[b], w_out[0]), b
            assert np.array_equal(pd[b], w_pd[0].astype(np.float32)), b
        else:
            same, f = check_sample_sequence(z64, vi.draft_probs[b], vi.draft_tokens[b],
                                            vi.uniforms[b], float(temps[b]), out[b], acc[b], pd[b])
            mism += not same
            flags += f
    assert mism <= flags
    return out, acc, pd


@pytest.mark.parametrize("cfg", [1, 2, 4])
def test_mixed_workloads(gpu, cfg):
    vi = synth.make_verify_inputs(synth.verify_config(cfg))
    temps = synth.make_temperatures(vi.spec.B, 100 + cfg)
    if cfg == 1:
        temps[:] = 0.7
    _mixed_parity(gpu, vi, temps)


@pytest.mark.parametrize("dtype,V", [("bf16", 1001), ("f32", 4099)])
def test_mixed_ragged_vocabulary(gpu, dtype, V):
    """A vocabulary that is not a multiple of 8 (the unvectorised kernels)."""
    from types import SimpleNamespace
    from tests.test_gpu_verify import _random_case
    B, K = 10, 4
    rng = np.random.default_rng(V)
    logits, q, d, u = _random_case(rng, B, K, V, dtype, T=0.8)
    vi = SimpleNamespace(logits=logits, draft_probs=q, draft_tokens=d, uniforms=u,
                         spec=SimpleNamespace(B=B, dtype=dtype))
    temps = np.array([0.0, 0.5, 0.7, 1.0, 1.3, 0.0, 0.8, 0.0, 2.0, 0.6], dtype=np.float32)
    _mixed_parity(gpu, vi, temps)


def test_every_sequence_mode_in_one_batch(gpu):
    # the mid-size verify batch (B=8, V=32000): every kind of temperature
    vi = synth.make_verify_inputs(synth.verify_config(2))
    temps = np.array([0.0, 0.5, 1.0, 0.0, 1.3, 0.7, 0.0, 2.0], dtype=np.float32)
    _mixed_parity(gpu, vi, temps)


def test_uniform_batches_match_single_mode_calls(gpu):
    vi = synth.make_verify_inputs(synth.verify_config(4))
    B = vi.spec.B
    z, q, d, u = dev(vi.logits), dev(vi.draft_probs), dev(vi.draft_tokens), dev(vi.uniforms)
    o1, a1, p1 = gpu.spec_verify_mixed(z, q, d, u, torch.full((B,), vi.temperature, device=DEV),
                                       want_draft_target_prob=True)
    o2, a2, p2 = gpu.spec_verify_sample(z, q, d, u, vi.temperature, want_draft_target_prob=True)
    o3, a3, p3 = gpu.spec_verify_mixed(z, q, d, u, torch.zeros(B, device=DEV),
                                       want_draft_target_prob=True)
    o4, a4 = gpu.spec_verify_greedy(z, d)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(a1, a2)
    assert torch.equal(p1.view(torch.int32), p2.view(torch.int32))
    assert torch.equal(o3, o4) and torch.equal(a3, a4)


def test_invalid_temperatures_are_greedy_and_flagged(gpu):
    vi = synth.make_verify_inputs(synth.verify_config(2))
    temps = np.array([0.7, -1.0, np.nan, np.inf, 1e-39, 1e-38, 0.0, 1.0], dtype=np.float32)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, acc, _ = gpu.spec_verify_mixed(dev(vi.logits), dev(vi.draft_probs), dev(vi.draft_tokens),
                                        dev(vi.uniforms), dev(temps), device_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) == gpu.DEVERR_TEMPERATURE
    out, acc = out.cpu().numpy(), acc.cpu().numpy()
    w_out, w_acc = oracle.verify_greedy(vi.logits, vi.spec.dtype, vi.draft_tokens)
    for b in (1, 2, 3, 4, 6):
        assert acc[b] == w_acc[b] and np.array_equal(out[b], w_out[b]), b
    # the clean workspace: a sampled call afterwards is unaffected
    _mixed_parity(gpu, vi, np.full(vi.spec.B, 0.9, np.float32))


@pytest.mark.parametrize("V", [1000, 5000, 40000])
def test_mixed_leaves_workspace_clear(gpu, V):
    """Greedy and sampled sequences in one batch leave the workspace all zero,
    with one draw workgroup per sequence (V = 1000 and 5000: rows of one and
    three CDF tiles kept in registers; the greedy sequences' workgroups stop
    after the scan) and with several (V = 40000, and the locate kernel)."""
    from tests.test_gpu_verify import _random_case
    rng = np.random.default_rng(V + 3)
    B, K = 12, 5
    logits, q, d, u = _random_case(rng, B, K, V, "f32", T=0.8)
    temps = np.array([0.0, 0.8, 0.0, 1.2, 0.5, 0.0, 0.7, 0.9, 0.0, 1.0, 0.0, 0.6], np.float32)
    ws = torch.zeros(gpu.spec_verify_workspace_bytes(B, K, V), dtype=torch.uint8, device=DEV)
    outs = []
    for _ in range(2):
        out, acc, _ = gpu.spec_verify_mixed(dev(logits), dev(q), dev(d), dev(u), dev(temps),
                                            workspace=ws)
        torch.cuda.synchronize()
        assert int(ws.count_nonzero().item()) == 0
        outs.append((out.cpu().numpy(), acc.cpu().numpy()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
    w_out, w_acc, _ = oracle.verify_mixed(logits, "f32", q, d, u, temps)
    greedy = temps == 0
    assert np.array_equal(outs[0][1][greedy], w_acc[greedy])
    assert np.array_equal(outs[0][0][greedy], w_out[greedy])
