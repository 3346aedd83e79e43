"""GPU: on-device acceptance metrics and the captured decode-step graph.

* spec_accept_metrics against oracle.metrics.counters, over several calls
  and more sequences than one workgroup covers, with out-of-range accept
  counts flagged and clamped.
* A step graph (verify, build, metrics) replayed several times with new
  inputs copied into its buffers and eager calls on other buffers in
  between: every replay must match the oracle on that replay's inputs (the
  verify outputs of every sequence, greedy ones exactly and sampled ones up
  to 1e-6 near ties; the build bit for bit), equal the eager step on the
  same inputs bit for bit, and the metrics must equal the oracle's counters
  of all replays.  Greedy, sampled and mixed graphs, and sampled and mixed
  graphs with q from the drafter logits.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.workloads import BuildSpec
from tests.gpu_util import DEV, check_sample_sequence, dev, host_bits

pytestmark = pytest.mark.gpu


def test_metrics_match_oracle(gpu):
    rng = np.random.default_rng(71)
    K = 7
    m = gpu.accept_metrics_buffer(K, DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    want = None
    for B in (1, 1000, 70_000):
        a = rng.integers(0, K + 1, size=B).astype(np.int32)
        gpu.spec_accept_metrics(dev(a), K, m, device_error=err)
        c = oracle.metrics.counters(a, K)
        want = c if want is None else oracle.metrics.accumulate(want, c)
    torch.cuda.synchronize()
    got = m.cpu().numpy()
    assert int(err.item()) == 0
    assert got[gpu.METRICS_STEPS] == want["steps"] == 3
    assert got[gpu.METRICS_ROUNDS] == want["rounds"]
    assert got[gpu.METRICS_PROPOSED] == want["proposed"]
    assert got[gpu.METRICS_ACCEPTED] == want["accepted"]
    assert got[gpu.METRICS_EMITTED] == want["emitted"]
    assert np.array_equal(got[gpu.METRICS_HIST:], want["hist"])
    s = gpu.acceptance_summary(m)
    r = oracle.metrics.rates(want)
    assert s["acceptance_length"] == r["acceptance_length"]
    assert s["draft_acceptance_rate"] == r["draft_acceptance_rate"]
    # out-of-range counts: flagged, clamped into [0, K]
    m2 = gpu.accept_metrics_buffer(3, DEV)
    gpu.spec_accept_metrics(dev(np.array([-2, 1, 5, 3], np.int32)), 3, m2, device_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) == gpu.DEVERR_ACCEPT_COUNT
    assert m2.cpu().numpy()[gpu.METRICS_HIST:].tolist() == [1, 1, 0, 2]


def _build_inputs(B, K, V):
    bi = synth.make_build_inputs(BuildSpec(0, B, K, 512, V, 16, 700, 16, 77, False))
    return dict(start_pos=dev(bi.start_pos), block_table=dev(bi.block_table),
                block_size=bi.spec.block_size, target_hidden=dev(bi.target_hidden),
                h_shared=dev(bi.h_shared), mask_token_id=bi.mask_token_id, host=bi)


def _replay_matches_oracle(mode, logits, dtype, q, d, u, T, temps, o, bi):
    """One replay's outputs against the oracle on the inputs it read: every
    sequence's verify outputs, then the build from those outputs bit for bit."""
    tok, acc, pd = o["tok"].cpu().numpy(), o["acc"].cpu().numpy(), o["pd"].cpu().numpy()
    B = logits.shape[0]
    if mode == "greedy":
        w_out, w_acc = oracle.verify_greedy(logits, dtype, d)
        assert np.array_equal(acc, w_acc) and np.array_equal(tok, w_out)
    for b in range(B if mode != "greedy" else 0):
        Tb = T if mode == "sample" else float(temps[b])
        if mode == "mixed" and oracle.mixed.is_greedy(temps[b]):
            w_out, w_acc, w_pd = oracle.verify_mixed(logits[b:b + 1], dtype, q[b:b + 1],
                                                     d[b:b + 1], u[b:b + 1], temps[b:b + 1])
            assert acc[b] == w_acc[0] and np.array_equal(tok[b], w_out[0]), b
            assert np.array_equal(pd[b], w_pd[0].astype(np.float32)), b
        else:
            check_sample_sequence(oracle.decode_logits(logits[b], dtype), q[b], d[b], u[b], Tb,
                                  tok[b], acc[b], pd[b])
    want = oracle.build_draft_batch(tok, acc, d, bi.start_pos, bi.block_table, bi.spec.block_size,
                                    bi.target_hidden, bi.h_shared, bi.mask_token_id)
    for key, v in o["build"].items():
        got = host_bits(v) if key == "hidden" else v.cpu().numpy()
        assert np.array_equal(got, want[key]), key


def _outputs(B, K, V, H):
    return dict(tok=torch.empty((B, K + 1), dtype=torch.int32, device=DEV),
                acc=torch.empty(B, dtype=torch.int32, device=DEV),
                pd=torch.empty((B, K), dtype=torch.float32, device=DEV),
                build={"input_ids": torch.empty(B * 2 * K, dtype=torch.int32, device=DEV),
                       "positions": torch.empty(B * 2 * K, dtype=torch.int64, device=DEV),
                       "slot_mapping": torch.empty(B * 2 * K, dtype=torch.int64, device=DEV),
                       "hidden": torch.empty((B * 2 * K, H), dtype=torch.bfloat16, device=DEV),
                       "sample_rows": torch.empty((B, K), dtype=torch.int32, device=DEV)})


def _eager(sv, mode, inp, b, o, ws, m):
    if mode == "greedy":
        sv.spec_verify_greedy(inp["z"], inp["d"], out_tokens=o["tok"], out_num_accepted=o["acc"],
                              workspace=ws)
    elif mode == "sample":
        sv.spec_verify_sample(inp["z"], inp["q"], inp["d"], inp["u"], inp["T"],
                              out_tokens=o["tok"], out_num_accepted=o["acc"],
                              out_draft_target_prob=o["pd"], workspace=ws)
    else:
        sv.spec_verify_mixed(inp["z"], inp["q"], inp["d"], inp["u"], inp["temps"],
                             out_tokens=o["tok"], out_num_accepted=o["acc"],
                             out_draft_target_prob=o["pd"], workspace=ws)
    sv.peagle_build_draft_batch(o["tok"], o["acc"], inp["d"], b["start_pos"], b["block_table"],
                                b["block_size"], b["target_hidden"], b["h_shared"],
                                b["mask_token_id"], outputs=o["build"])
    sv.spec_accept_metrics(o["acc"], inp["d"].shape[1], m)


@pytest.mark.parametrize("mode", ["sample", "greedy", "mixed"])
def test_step_graph_replays_match_eager(gpu, mode):
    vi = synth.make_verify_inputs(synth.verify_config(2))
    B, K, V = vi.spec.B, vi.spec.K, vi.spec.V
    rng = np.random.default_rng(72)
    temps = np.array([0.0, 0.5, 1.0, 0.0, 1.3, 0.7, 0.0, 2.0], dtype=np.float32)
    inp = dict(z=dev(vi.logits), q=dev(vi.draft_probs), d=dev(vi.draft_tokens),
               u=dev(vi.uniforms), T=vi.temperature, temps=dev(temps))
    b = _build_inputs(B, K, V)
    bi = b.pop("host")
    og, oe = _outputs(B, K, V, 512), _outputs(B, K, V, 512)
    ws_g = torch.zeros(gpu.spec_verify_workspace_bytes(B, K, V), dtype=torch.uint8, device=DEV)
    ws_e = torch.zeros_like(ws_g)
    mg, me = gpu.accept_metrics_buffer(K, DEV), gpu.accept_metrics_buffer(K, DEV)
    verify = dict(target_logits=inp["z"], draft_tokens=inp["d"], out_tokens=og["tok"],
                  out_num_accepted=og["acc"], workspace=ws_g)
    if mode != "greedy":
        verify.update(draft_probs=inp["q"], uniforms=inp["u"], out_draft_target_prob=og["pd"])
    if mode == "sample":
        verify["temperature"] = vi.temperature
    if mode == "mixed":
        verify["temperatures"] = inp["temps"]
    graph = gpu.StepGraph(mode, verify, dict(b, outputs=og["build"]), metrics=mg)
    accs = []
    for rep in range(4):
        # new inputs in the captured buffers: fresh uniforms and drafts
        u_new = rng.random((B, K + 1), dtype=np.float32)
        d_new = vi.draft_tokens.copy()
        if rep % 2:
            d_new[:, rep % K] = rng.integers(0, V, size=B)
        inp["u"].copy_(dev(u_new))
        inp["d"].copy_(dev(d_new))
        graph.launch()
        torch.cuda.synchronize()
        _replay_matches_oracle(mode, vi.logits, vi.spec.dtype, vi.draft_probs, d_new, u_new,
                               vi.temperature, temps, og, bi)
        _eager(gpu, mode, inp, b, oe, ws_e, me)
        torch.cuda.synchronize()
        assert torch.equal(og["tok"], oe["tok"]) and torch.equal(og["acc"], oe["acc"]), rep
        if mode != "greedy":
            assert torch.equal(og["pd"].view(torch.int32), oe["pd"].view(torch.int32)), rep
        for k in og["build"]:
            assert torch.equal(og["build"][k], oe["build"][k]), (rep, k)
        accs.append(oe["acc"].cpu().numpy())
    want = oracle.metrics.counters(accs[0], K)
    for a in accs[1:]:
        want = oracle.metrics.accumulate(want, oracle.metrics.counters(a, K))
    assert torch.equal(mg, me)
    got = mg.cpu().numpy()
    assert got[gpu.METRICS_ACCEPTED] == want["accepted"] and got[gpu.METRICS_STEPS] == 4
    assert np.array_equal(got[gpu.METRICS_HIST:], want["hist"])
    graph.close()


def test_step_graph_argument_errors(gpu):
    z = torch.zeros((2, 4, 64), dtype=torch.float32, device=DEV)
    d = torch.zeros((2, 3), dtype=torch.int32, device=DEV)
    verify = dict(target_logits=z, draft_tokens=d,
                  out_tokens=torch.empty((2, 4), dtype=torch.int32, device=DEV),
                  out_num_accepted=torch.empty(2, dtype=torch.int32, device=DEV),
                  workspace=torch.zeros(16, dtype=torch.uint8, device=DEV))    # too small
    with pytest.raises(gpu.SpecVerifyError):
        gpu.StepGraph("greedy", verify)
    verify["workspace"] = torch.zeros(gpu.spec_verify_workspace_bytes(2, 3, 64),
                                      dtype=torch.uint8, device=DEV)
    g = gpu.StepGraph("greedy", verify)
    g.launch()
    torch.cuda.synchronize()
    # all-zero logits: every argmax is token 0, so all-zero drafts are all accepted
    assert verify["out_num_accepted"].cpu().tolist() == [3, 3]
    assert verify["out_tokens"].cpu().tolist() == [[0, 0, 0, 0], [0, 0, 0, 0]]
    g.close()


def test_metrics_at_max_drafts(gpu):
    rng = np.random.default_rng(73)
    K = 63
    a = rng.integers(0, K + 1, size=5000).astype(np.int32)
    m = gpu.accept_metrics_buffer(K, DEV)
    gpu.spec_accept_metrics(dev(a), K, m)
    torch.cuda.synchronize()
    want = oracle.metrics.counters(a, K)
    got = m.cpu().numpy()
    assert np.array_equal(got[gpu.METRICS_HIST:], want["hist"])
    assert got[gpu.METRICS_ACCEPTED] == want["accepted"]


@pytest.mark.parametrize("B,V,dtype", [(300, 40000, "bf16"), (900, 40001, "f32"),
                                        (900, 5000, "f32")])
def test_step_graph_one_draw_workgroup_per_sequence(gpu, B, V, dtype):
    """Sampled step graphs whose draw runs one workgroup per sequence and
    draws the token itself (B = 300, V = 40000: 512-thread workgroups; B =
    900, V = 40001: 256-thread workgroups; V = 5000: the row's three CDF tiles
    kept in registers): every replay with new uniforms matches the oracle and
    equals the eager step."""
    from tests.test_gpu_verify import _random_case
    K, T = 3, 0.9
    rng = np.random.default_rng(B)
    logits, q, d, u = _random_case(rng, B, K, V, dtype, T=T)
    inp = dict(z=dev(logits), q=dev(q), d=dev(d), u=dev(u), T=T)
    b = _build_inputs(B, K, V)
    bi = b.pop("host")
    og, oe = _outputs(B, K, V, 512), _outputs(B, K, V, 512)
    ws_g = torch.zeros(gpu.spec_verify_workspace_bytes(B, K, V), dtype=torch.uint8, device=DEV)
    ws_e = torch.zeros_like(ws_g)
    mg, me = gpu.accept_metrics_buffer(K, DEV), gpu.accept_metrics_buffer(K, DEV)
    verify = dict(target_logits=inp["z"], draft_tokens=inp["d"], out_tokens=og["tok"],
                  out_num_accepted=og["acc"], workspace=ws_g, draft_probs=inp["q"],
                  uniforms=inp["u"], out_draft_target_prob=og["pd"], temperature=T)
    graph = gpu.StepGraph("sample", verify, dict(b, outputs=og["build"]), metrics=mg)
    for rep in range(3):
        u_new = rng.random((B, K + 1), dtype=np.float32)
        inp["u"].copy_(dev(u_new))
        graph.launch()
        torch.cuda.synchronize()
        _replay_matches_oracle("sample", logits, dtype, q, d, u_new, T, None, og, bi)
        _eager(gpu, "sample", inp, b, oe, ws_e, me)
        torch.cuda.synchronize()
        assert torch.equal(og["tok"], oe["tok"]) and torch.equal(og["acc"], oe["acc"]), rep
        assert torch.equal(og["pd"].view(torch.int32), oe["pd"].view(torch.int32)), rep
        for k in og["build"]:
            assert torch.equal(og["build"][k], oe["build"][k]), (rep, k)
    assert torch.equal(mg, me)
    assert int(ws_g.count_nonzero().item()) == 0
    graph.close()


@pytest.mark.parametrize("mode", ["sample", "mixed"])
def test_step_graph_lq_replays_match_oracle(gpu, mode):
    """Step graphs whose verify recomputes q from the drafter logits (sampled,
    with the drafter rows gathered through a row index; mixed, drafted at the
    requests' own temperatures).  Before each replay the drafter sampling
    writes new draft tokens and row descriptors into the captured buffers
    (fresh drafter uniforms) and new verify uniforms are copied in.  Every
    replay matches the oracle (q from oracle.draft.draft_probs of the drafter
    rows; the build bit for bit) and equals the eager step on the dense q of
    the same drafting bit for bit; the metrics equal the eager ones."""
    vi = synth.make_verify_inputs(synth.verify_config(2))       # B=8, K=5, V=32000 fp32
    B, K, V, dt = vi.spec.B, vi.spec.K, vi.spec.V, vi.spec.dtype
    rng = np.random.default_rng(74)
    base = oracle.decode_logits(vi.logits[:, :K].reshape(B * K, V), dt)
    zd = (base + rng.standard_normal(base.shape)).astype(np.float32)
    zd[~np.isfinite(base)] = base[~np.isfinite(base)]
    perm = rng.permutation(B * K).astype(np.int32).reshape(B, K) if mode == "sample" else None
    if perm is not None:                 # drafter row (b, k) stored at perm[b, k]
        stored = np.empty_like(zd)
        stored[perm.reshape(-1)] = zd
        zd = stored
    if dt == "bf16":
        zd = synth.f32_to_bf16_bits(zd)
    temps = np.array([0.0, 0.5, 1.0, 0.0, 1.3, 0.7, 0.0, 2.0], dtype=np.float32)
    Td = 0.8
    oq = oracle.draft.draft_probs(zd, dt, Td, B, K, row_index=perm,
                                  temperatures=temps if mode == "mixed" else None)
    z_t, zd_t, temps_t = dev(vi.logits), dev(zd), dev(temps)
    rows_t = None if perm is None else dev(perm)
    d_t = torch.empty((B, K), dtype=torch.int32, device=DEV)
    desc_t = torch.empty((B, K, 4), dtype=torch.int32, device=DEV)
    q_e = torch.empty((B, K, V), dtype=torch.float32, device=DEV)
    u_t = torch.empty((B, K + 1), dtype=torch.float32, device=DEV)
    ud_t = torch.empty((B, K), dtype=torch.float32, device=DEV)

    def draft(ud):
        ud_t.copy_(dev(ud))
        gpu.spec_draft_sample(zd_t, K, Td, uniforms=ud_t, row_index=rows_t,
                              temperatures=temps_t if mode == "mixed" else None,
                              out_draft_tokens=d_t, out_draft_probs=q_e, out_row_desc=desc_t)

    draft(rng.random((B, K), dtype=np.float32))
    b = _build_inputs(B, K, V)
    bi = b.pop("host")
    og, oe = _outputs(B, K, V, 512), _outputs(B, K, V, 512)
    ws_g = torch.zeros(gpu.spec_verify_workspace_bytes(B, K, V), dtype=torch.uint8, device=DEV)
    ws_e = torch.zeros_like(ws_g)
    mg, me = gpu.accept_metrics_buffer(K, DEV), gpu.accept_metrics_buffer(K, DEV)
    verify = dict(target_logits=z_t, draft_tokens=d_t, out_tokens=og["tok"],
                  out_num_accepted=og["acc"], workspace=ws_g, uniforms=u_t,
                  out_draft_target_prob=og["pd"], drafter_logits=zd_t, drafter_desc=desc_t,
                  drafter_rows=rows_t)
    if mode == "sample":
        verify["temperature"] = vi.temperature
    else:
        verify["temperatures"] = temps_t
    graph = gpu.StepGraph(mode, verify, dict(b, outputs=og["build"]), metrics=mg)
    inp = dict(z=z_t, q=q_e, d=d_t, u=u_t, T=vi.temperature, temps=temps_t)
    for rep in range(4):
        draft(rng.random((B, K), dtype=np.float32))
        u_new = rng.random((B, K + 1), dtype=np.float32)
        u_t.copy_(dev(u_new))
        graph.launch()
        torch.cuda.synchronize()
        d_host = d_t.cpu().numpy()
        _replay_matches_oracle(mode, vi.logits, dt, oq, d_host, u_new, vi.temperature, temps,
                               og, bi)
        _eager(gpu, mode, inp, b, oe, ws_e, me)
        torch.cuda.synchronize()
        assert torch.equal(og["tok"], oe["tok"]) and torch.equal(og["acc"], oe["acc"]), rep
        assert torch.equal(og["pd"].view(torch.int32), oe["pd"].view(torch.int32)), rep
        for k in og["build"]:
            assert torch.equal(og["build"][k], oe["build"][k]), (rep, k)
    assert torch.equal(mg, me)
    assert int(ws_g.count_nonzero().item()) == 0
    graph.close()


@pytest.mark.parametrize("mode", ["sample", "greedy", "mixed"])
def test_step_graph_early_exit(gpu, mode):
    """A step graph capturing the early-exit verify: every replay (new
    uniforms and drafts copied in) matches the oracle on its inputs and
    equals the eager full step in tokens, accept counts and the build;
    p_k(d_k) equals the full step's up to the first rejection and is 0 past
    it; the metrics equal the eager ones."""
    vi = synth.make_verify_inputs(synth.verify_config(2))
    B, K, V = vi.spec.B, vi.spec.K, vi.spec.V
    rng = np.random.default_rng(76)
    temps = np.array([0.0, 0.5, 1.0, 0.0, 1.3, 0.7, 0.0, 2.0], dtype=np.float32)
    inp = dict(z=dev(vi.logits), q=dev(vi.draft_probs), d=dev(vi.draft_tokens),
               u=dev(vi.uniforms), T=vi.temperature, temps=dev(temps))
    b = _build_inputs(B, K, V)
    bi = b.pop("host")
    og, oe = _outputs(B, K, V, 512), _outputs(B, K, V, 512)
    ws_g = torch.zeros(gpu.spec_verify_workspace_bytes(B, K, V), dtype=torch.uint8, device=DEV)
    ws_e = torch.zeros_like(ws_g)
    mg, me = gpu.accept_metrics_buffer(K, DEV), gpu.accept_metrics_buffer(K, DEV)
    verify = dict(target_logits=inp["z"], draft_tokens=inp["d"], out_tokens=og["tok"],
                  out_num_accepted=og["acc"], workspace=ws_g)
    if mode != "greedy":
        verify.update(draft_probs=inp["q"], uniforms=inp["u"], out_draft_target_prob=og["pd"])
    if mode == "sample":
        verify["temperature"] = vi.temperature
    if mode == "mixed":
        verify["temperatures"] = inp["temps"]
    graph = gpu.StepGraph(mode, verify, dict(b, outputs=og["build"]), metrics=mg,
                          early_exit=True)
    for rep in range(3):
        u_new = rng.random((B, K + 1), dtype=np.float32)
        d_new = vi.draft_tokens.copy()
        if rep % 2:
            d_new[:, rep % K] = rng.integers(0, V, size=B)
        inp["u"].copy_(dev(u_new))
        inp["d"].copy_(dev(d_new))
        graph.launch()
        torch.cuda.synchronize()
        _eager(gpu, mode, inp, b, oe, ws_e, me)
        torch.cuda.synchronize()
        # the replay's tokens, counts and build against the oracle (p_k(d_k)
        # past the first rejection is not computed here: the full step's)
        _replay_matches_oracle(mode, vi.logits, vi.spec.dtype, vi.draft_probs, d_new, u_new,
                               vi.temperature, temps, dict(og, pd=oe["pd"]), bi)
        assert torch.equal(og["tok"], oe["tok"]) and torch.equal(og["acc"], oe["acc"]), rep
        if mode != "greedy":
            keep = torch.arange(K, device=DEV)[None, :] <= oe["acc"].long()[:, None]
            want = torch.where(keep, oe["pd"], torch.zeros_like(oe["pd"]))
            assert torch.equal(og["pd"].view(torch.int32), want.view(torch.int32)), rep
        for k in og["build"]:
            assert torch.equal(og["build"][k], oe["build"][k]), (rep, k)
    assert torch.equal(mg, me)
    assert int(ws_g.count_nonzero().item()) == 0
    graph.close()
