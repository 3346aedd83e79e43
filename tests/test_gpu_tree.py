"""GPU parity: spec_verify_tree against the draft-tree oracle.

Greedy trees are compared exactly (tokens, node path, accept length).
Sampled trees: the GPU's (path, new token) must be the oracle's, or one the
oracle lists when a test lies within 1e-6 of its threshold or the final draw
within 1e-6 of a CDF boundary (oracle.tree.tree_outcomes).  Covered: random,
static and chain trees; fp32 and bf16, each also with a vocabulary that is
not a multiple of 8; V up to 151936; a root without children; invalid
nodes; determinism and a clean workspace.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import TREE_CONFIGS, make_tree_inputs
from tests.gpu_util import DEV, TIE_TOL, dev

pytestmark = pytest.mark.gpu


def _run(sv, ti, T, parents=None, tokens=None):
    par = ti.parents if parents is None else parents
    tok = ti.tokens if tokens is None else tokens
    out, path, acc = sv.spec_verify_tree(dev(ti.logits), dev(par), dev(tok), T,
                                         draft_probs=dev(ti.draft_probs), uniforms=dev(ti.uniforms))
    torch.cuda.synchronize()
    return out.cpu().numpy(), path.cpu().numpy(), acc.cpu().numpy()


def _check_greedy(ti, out, path, acc, parents=None, tokens=None):
    par = ti.parents if parents is None else parents
    tok = ti.tokens if tokens is None else tokens
    for b in range(ti.spec.B):
        z64 = oracle.decode_logits(ti.logits[b], ti.spec.dtype)
        a, o, n = oracle.tree.verify_tree_greedy_seq(z64, par[b], tok[b])
        assert acc[b] == a and np.array_equal(out[b], o) and np.array_equal(path[b], n), b


def _check_sample(ti, T, out, path, acc, max_flag_frac=0.02):
    flags = 0
    for b in range(ti.spec.B):
        z64 = oracle.decode_logits(ti.logits[b], ti.spec.dtype)
        a = int(acc[b])
        got = (tuple(int(x) for x in path[b, :a]), int(out[b, a]))
        canon, allowed = oracle.tree.tree_outcomes(z64, ti.draft_probs[b], ti.parents[b],
                                                   ti.tokens[b], ti.uniforms[b], T, tol=TIE_TOL)
        assert got in allowed, (b, got, canon, allowed)
        flags += got != canon
        # the emitted tokens are the path's tokens
        assert all(out[b, j] == ti.tokens[b, path[b, j] - 1] for j in range(a))
        assert np.all(out[b, a + 1:] == -1) and np.all(path[b, a:] == -1)
    assert flags <= max(2, max_flag_frac * ti.spec.B)


@pytest.mark.parametrize("name", ["tree-tiny", "tree-mid", "tree-large"])
def test_tree_workloads(gpu, name):
    ti = make_tree_inputs(TREE_CONFIGS[name])
    _check_greedy(ti, *_run(gpu, ti, 0.0))
    T = ti.temperature
    _check_sample(ti, T, *_run(gpu, ti, T))


def test_chain_tree_matches_chain_verify(gpu):
    vi = synth.make_verify_inputs(synth.verify_config(2))
    B, K, V = vi.spec.B, vi.spec.K, vi.spec.V
    par = np.broadcast_to(np.arange(K, dtype=np.int32), (B, K)).copy()
    q = np.concatenate([vi.draft_probs, np.full((B, 1, V), 1.0 / V, np.float32)], axis=1)
    u = np.concatenate([vi.uniforms[:, K:], vi.uniforms[:, :K]], axis=1)
    out, path, acc = gpu.spec_verify_tree(dev(vi.logits), dev(par), dev(vi.draft_tokens),
                                          vi.temperature, draft_probs=dev(q), uniforms=dev(u))
    o2, a2, _ = gpu.spec_verify_sample(dev(vi.logits), dev(vi.draft_probs), dev(vi.draft_tokens),
                                       dev(vi.uniforms), vi.temperature)
    og, pg, ag = gpu.spec_verify_tree(dev(vi.logits), dev(par), dev(vi.draft_tokens), 0.0)
    o3, a3 = gpu.spec_verify_greedy(dev(vi.logits), dev(vi.draft_tokens))
    torch.cuda.synchronize()
    assert torch.equal(acc, a2) and torch.equal(out, o2)
    assert torch.equal(ag, a3) and torch.equal(og, o3)
    p = path.cpu().numpy()
    for b, a in enumerate(acc.cpu().numpy()):
        assert p[b, :a].tolist() == list(range(1, a + 1))


def test_root_only_and_invalid_nodes(gpu):
    ti = make_tree_inputs(TREE_CONFIGS["tree-tiny"])
    B, N, V = ti.spec.B, ti.spec.N, ti.spec.V
    # N = 0: greedy emits the root's argmax, sampled draws from the root row
    z0 = ti.logits[:, :1]
    out, path, acc = gpu.spec_verify_tree(dev(z0), dev(np.zeros((B, 0), np.int32)),
                                          dev(np.zeros((B, 0), np.int32)), 0.0)
    torch.cuda.synchronize()
    assert acc.cpu().tolist() == [0] * B
    want = [oracle.first_argmax(z0[b, 0].astype(np.float64)) for b in range(B)]
    assert out.cpu().numpy()[:, 0].tolist() == want
    # invalid nodes: flagged and treated as absent
    par = ti.parents.copy()
    tok = ti.tokens.copy()
    par[0, 2] = 5            # node 3's parent does not precede it
    tok[1, 0] = V + 4        # node 1's token is outside the vocabulary
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, path, acc = gpu.spec_verify_tree(dev(ti.logits), dev(par), dev(tok), 0.0,
                                          device_error=err)
    torch.cuda.synchronize()
    assert int(err.item()) == gpu.DEVERR_TREE
    par_o = par.copy()
    tok_o = tok.copy()
    # the oracle's reading of an absent node: it is nobody's child; mark it with
    # a parent no node can have (itself) after validation, by removing it
    for b, i in [(0, 2), (1, 0)]:
        par_o[b, i] = -1
    out, path, acc = out.cpu().numpy(), path.cpu().numpy(), acc.cpu().numpy()
    for b in range(B):
        z64 = oracle.decode_logits(ti.logits[b], ti.spec.dtype)
        cur, k = 0, 0
        while True:
            g = oracle.first_argmax(z64[cur])
            kids = [i for i in range(1, N + 1) if par_o[b, i - 1] == cur and tok_o[b, i - 1] == g]
            if not kids:
                assert out[b, k] == g and acc[b] == k
                break
            assert path[b, k] == kids[0]
            cur, k = kids[0], k + 1


def test_determinism_and_clean_workspace(gpu):
    ti = make_tree_inputs(TREE_CONFIGS["tree-mid"])
    B, N, V = ti.spec.B, ti.spec.N, ti.spec.V
    ws = torch.zeros(gpu.spec_verify_workspace_bytes(B, N, V), dtype=torch.uint8, device=DEV)
    args = (dev(ti.logits), dev(ti.parents), dev(ti.tokens), ti.temperature)
    kw = dict(draft_probs=dev(ti.draft_probs), uniforms=dev(ti.uniforms), workspace=ws)
    r1 = gpu.spec_verify_tree(*args, **kw)
    r2 = gpu.spec_verify_tree(*args, **kw)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(r1, r2))
    assert int(ws.count_nonzero().item()) == 0


def test_max_nodes_random_trees(gpu):
    """N = 63 nodes (the limit) with a vocabulary that is not a multiple of 8."""
    from synth.workloads import TreeSpec
    spec = TreeSpec("tree-max", 3, 63, 4099, "f32", 2.0, "none", 1.0, 0.5, 1.0, "random", (), 25)
    ti = make_tree_inputs(spec, workers=1)
    _check_greedy(ti, *_run(gpu, ti, 0.0))
    _check_sample(ti, 1.0, *_run(gpu, ti, 1.0))


def test_bf16_ragged_vocabulary_trees(gpu):
    """bf16 logits with a vocabulary that is not a multiple of 8."""
    from synth.workloads import TreeSpec
    spec = TreeSpec("tree-ragged", 6, 9, 30011, "bf16", 3.0, "zipf-head", 0.7, 1.0, 0.7,
                    "static", (3, 2), 26)
    ti = make_tree_inputs(spec, workers=1)
    _check_greedy(ti, *_run(gpu, ti, 0.0))
    _check_sample(ti, ti.temperature, *_run(gpu, ti, ti.temperature))
