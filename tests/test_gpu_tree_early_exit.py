"""GPU: the early-exit tree verify (spec_verify_tree_early_exit,
spec_verify_tree_lq_early_exit), whose walk computes the statistics of the
rows it visits instead of reading the row kernel's statistics of every row.

Greedy walks must equal the full call and the oracle exactly.  Sampled walks
add a row's exponentials in another order than the row kernel, so they are
checked against the oracle with the 1e-6 near-tie rule (oracle.tree.
tree_outcomes) and must agree with the full call on all but a few flagged
trees.  The drafter-logit form must equal the dense form bit for bit on the
same drafting (both walks compute q and the statistics the same way).
Covered: the tiny, mid and large tree workloads, 63-node random trees, bf16
with a vocabulary that is not a multiple of 8, a root without children,
invalid nodes (same flags), and a workspace left untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import TREE_CONFIGS, make_tree_inputs
from synth.workloads import TreeSpec
from tests.gpu_util import DEV, TIE_TOL, dev
from tests.test_gpu_tree import _check_greedy, _check_sample

pytestmark = pytest.mark.gpu


def _both(sv, ti, T, parents=None, tokens=None, err=None):
    par = dev(ti.parents if parents is None else parents)
    tok = dev(ti.tokens if tokens is None else tokens)
    kw = dict(draft_probs=dev(ti.draft_probs), uniforms=dev(ti.uniforms)) if T > 0 else {}
    B, N, V = ti.spec.B, ti.spec.N, ti.spec.V
    ws = torch.zeros(sv.spec_verify_workspace_bytes(B, N, V), dtype=torch.uint8, device=DEV)
    errs = [torch.zeros(1, dtype=torch.int32, device=DEV) for _ in range(2)]
    full = sv.spec_verify_tree(dev(ti.logits), par, tok, T, device_error=errs[0], **kw)
    ee = sv.spec_verify_tree_early_exit(dev(ti.logits), par, tok, T, workspace=ws,
                                        device_error=errs[1], **kw)
    torch.cuda.synchronize()
    assert int(errs[0].item()) == int(errs[1].item())
    assert int(ws.count_nonzero().item()) == 0
    return ([x.cpu().numpy() for x in full], [x.cpu().numpy() for x in ee],
            int(errs[1].item()))


def _agree(full, ee, max_diff):
    same = np.array([np.array_equal(full[0][b], ee[0][b]) and np.array_equal(full[1][b], ee[1][b])
                     for b in range(full[0].shape[0])])
    assert np.array_equal(full[2][same], ee[2][same])
    assert (~same).sum() <= max_diff


@pytest.mark.parametrize("name", ["tree-tiny", "tree-mid", "tree-large"])
def test_workloads(gpu, name):
    ti = make_tree_inputs(TREE_CONFIGS[name])
    full, ee, _ = _both(gpu, ti, 0.0)
    for x, y in zip(full, ee):
        assert np.array_equal(x, y)
    _check_greedy(ti, *ee)
    T = ti.temperature
    full, ee, _ = _both(gpu, ti, T)
    _check_sample(ti, T, *ee)
    _agree(full, ee, max(2, 0.02 * ti.spec.B))


def test_max_nodes_and_ragged_bf16(gpu):
    for spec in (TreeSpec("tree-max", 3, 63, 4099, "f32", 2.0, "none", 1.0, 0.5, 1.0, "random",
                          (), 25),
                 TreeSpec("tree-ragged", 6, 9, 30011, "bf16", 3.0, "zipf-head", 0.7, 1.0, 0.7,
                          "static", (3, 2), 26)):
        ti = make_tree_inputs(spec, workers=1)
        full, ee, _ = _both(gpu, ti, 0.0)
        for x, y in zip(full, ee):
            assert np.array_equal(x, y)
        full, ee, _ = _both(gpu, ti, spec.temperature)
        _check_sample(ti, spec.temperature, *ee)


def test_root_only_and_invalid_nodes(gpu):
    ti = make_tree_inputs(TREE_CONFIGS["tree-tiny"])
    B, N, V = ti.spec.B, ti.spec.N, ti.spec.V
    z0 = ti.logits[:, :1]
    for T in (0.0, 0.8):
        kw = dict(draft_probs=dev(ti.draft_probs[:, :1]), uniforms=dev(ti.uniforms[:, :1])) \
            if T > 0 else {}
        out, path, acc = gpu.spec_verify_tree_early_exit(
            dev(z0), dev(np.zeros((B, 0), np.int32)), dev(np.zeros((B, 0), np.int32)), T, **kw)
        torch.cuda.synchronize()
        assert acc.cpu().tolist() == [0] * B
        if T == 0.0:
            want = [oracle.first_argmax(z0[b, 0].astype(np.float64)) for b in range(B)]
            assert out.cpu().numpy()[:, 0].tolist() == want
    par = ti.parents.copy()
    tok = ti.tokens.copy()
    par[0, 2] = 5                      # node 3's parent does not precede it
    tok[1, 0] = V + 4                  # node 1's token is outside the vocabulary
    for T in (0.0, ti.temperature):
        full, ee, err = _both(gpu, ti, T, parents=par, tokens=tok)
        assert err == gpu.DEVERR_TREE
        if T == 0.0:
            for x, y in zip(full, ee):
                assert np.array_equal(x, y)


def test_drafter_logit_form(gpu):
    """spec_verify_tree_lq_early_exit equals spec_verify_tree_early_exit on the
    dense q and descriptors of one drafting, bit for bit, and the oracle."""
    ti = make_tree_inputs(TREE_CONFIGS["tree-large"])
    B, N, V = ti.spec.B, ti.spec.N, ti.spec.V
    n = B * (N + 1)
    rng = np.random.default_rng(17)
    z = oracle.decode_logits(ti.logits.reshape(n, V), ti.spec.dtype).astype(np.float32)
    zd = z + rng.standard_normal(z.shape).astype(np.float32)
    zd[~np.isfinite(z)] = z[~np.isfinite(z)]
    zd = synth.f32_to_bf16_bits(zd) if ti.spec.dtype == "bf16" else zd
    rows = rng.permutation(n).astype(np.int32).reshape(B, N + 1)
    ud = rng.random((n, 1), dtype=np.float32)
    _, q, desc = gpu.spec_draft_sample(dev(zd), 1, 0.7, uniforms=dev(ud),
                                       row_index=dev(rows.reshape(n, 1)), want_row_desc=True)
    T = ti.temperature
    par, tok, u, zt = dev(ti.parents), dev(ti.tokens), dev(ti.uniforms), dev(ti.logits)
    dense = gpu.spec_verify_tree_early_exit(zt, par, tok, T, draft_probs=q.view(B, N + 1, V),
                                            uniforms=u)
    lq = gpu.spec_verify_tree_lq_early_exit(zt, dev(zd), desc.view(B, N + 1, 4), par, tok, u, T,
                                            drafter_rows=dev(rows))
    full = gpu.spec_verify_tree_lq(zt, dev(zd), desc.view(B, N + 1, 4), par, tok, u, T,
                                   drafter_rows=dev(rows))
    torch.cuda.synchronize()
    for x, y in zip(dense, lq):
        assert torch.equal(x, y)
    _agree([x.cpu().numpy() for x in full], [x.cpu().numpy() for x in lq], max(2, 0.02 * B))
    out, path, acc = (x.cpu().numpy() for x in lq)
    flags = 0
    for b in range(B):
        qrows = np.stack([oracle.draft.draft_distribution(
            oracle.decode_logits(zd[int(rows[b, m])], ti.spec.dtype), float(np.float32(0.7)))
            for m in range(N + 1)])
        z64 = oracle.decode_logits(ti.logits[b], ti.spec.dtype)
        a = int(acc[b])
        got = (tuple(int(x) for x in path[b, :a]), int(out[b, a]))
        canon, allowed = oracle.tree.tree_outcomes(z64, qrows, ti.parents[b], ti.tokens[b],
                                                   ti.uniforms[b], T, tol=TIE_TOL)
        assert got in allowed, (b, got, canon, allowed)
        flags += got != canon
    assert flags <= max(2, 0.02 * B)
