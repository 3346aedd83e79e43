"""GPU: sampled tree verification with q recomputed from the drafter logits.

spec_draft_sample drafts one row per tree node (K = 1 over B*(N+1) rows) and
writes, for each, the dense q and the row descriptor; spec_verify_tree on the
dense q and spec_verify_tree_lq on the drafter logits + descriptors must then
agree bit for bit (tokens, node path, accept length).  The lq results are
also checked against the oracle: q of node n from oracle.draft's drafter
distribution of its drafter row, then oracle.tree.tree_outcomes with the
1e-6 near-tie tolerance.  Covered: V=151936 bf16 trees; fp32 trees with
drafter rows gathered through a row index, greedy-drafted nodes and an
invalid drafter row (flagged, q = 0 as the dense path's all-zero row); a
bf16 vocabulary that is not a multiple of 8; a root without children; trees
of 63 nodes (the limit) and an empty batch.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import TREE_CONFIGS, make_tree_inputs
from tests.gpu_util import DEV, TIE_TOL, dev

pytestmark = pytest.mark.gpu


def _drafter_rows(ti, seed, scale=1.0):
    """Stand-in drafter logits: the target rows plus seeded noise, in the
    target's dtype, one row per node (row b*(N+1) + n)."""
    B, N, V = ti.spec.B, ti.spec.N, ti.spec.V
    rng = np.random.default_rng(seed)
    z = oracle.decode_logits(ti.logits.reshape(B * (N + 1), V), ti.spec.dtype).astype(np.float32)
    zd = z + (scale * rng.standard_normal(z.shape)).astype(np.float32)
    zd[~np.isfinite(z)] = z[~np.isfinite(z)]
    return synth.f32_to_bf16_bits(zd) if ti.spec.dtype == "bf16" else zd


def _run(sv, ti, zd, Td, rows=None, temps=None, parents=None, err=None):
    B, N, V = ti.spec.B, ti.spec.N, ti.spec.V
    n = B * (N + 1)
    ud = np.random.default_rng(5).random((n, 1), dtype=np.float32)
    zd_t = dev(zd)
    rows_t = None if rows is None else dev(rows.reshape(n, 1))
    _, q, desc = sv.spec_draft_sample(zd_t, 1, Td, uniforms=dev(ud), row_index=rows_t,
                                      temperatures=None if temps is None else dev(temps),
                                      want_row_desc=True)
    par = dev(ti.parents if parents is None else parents)
    tok, u, z = dev(ti.tokens), dev(ti.uniforms), dev(ti.logits)
    T = ti.temperature
    dense = sv.spec_verify_tree(z, par, tok, T, draft_probs=q.view(B, N + 1, V), uniforms=u)
    lq = sv.spec_verify_tree_lq(z, zd_t, desc.view(B, N + 1, 4), par, tok, u, T,
                                drafter_rows=None if rows is None else dev(rows),
                                device_error=err)
    torch.cuda.synchronize()
    for x, y in zip(dense, lq):
        assert torch.equal(x, y)
    return tuple(x.cpu().numpy() for x in lq)


def _check_oracle(ti, zd, Td, out, path, acc, rows=None, temps=None, parents=None, skip=()):
    B, N, V = ti.spec.B, ti.spec.N, ti.spec.V
    par = ti.parents if parents is None else parents
    flags = 0
    for b in range(B):
        if b in skip:
            continue
        qrows = np.empty((N + 1, V))
        for n in range(N + 1):
            j = b * (N + 1) + n
            r = j if rows is None else int(rows[b, n])
            Tn = float(np.float32(Td if temps is None else temps[j]))
            qrows[n] = oracle.draft.draft_distribution(
                oracle.decode_logits(zd[r], ti.spec.dtype), Tn)
        z64 = oracle.decode_logits(ti.logits[b], ti.spec.dtype)
        a = int(acc[b])
        got = (tuple(int(x) for x in path[b, :a]), int(out[b, a]))
        canon, allowed = oracle.tree.tree_outcomes(z64, qrows, par[b], ti.tokens[b],
                                                   ti.uniforms[b], ti.temperature, tol=TIE_TOL)
        assert got in allowed, (b, got, canon, allowed)
        flags += got != canon
    assert flags <= max(2, 0.02 * B)


@pytest.mark.parametrize("name", ["tree-large"])
def test_tree_lq_matches_dense_and_oracle(gpu, name):
    ti = make_tree_inputs(TREE_CONFIGS[name])
    zd = _drafter_rows(ti, 17)
    out, path, acc = _run(gpu, ti, zd, 0.7)
    _check_oracle(ti, zd, 0.7, out, path, acc)
    assert acc.mean() > 0.3                # the stand-in drafter agrees often enough


def test_tree_lq_gathered_greedy_and_invalid_rows(gpu):
    ti = make_tree_inputs(TREE_CONFIGS["tree-mid"])               # fp32, V=32000
    B, N, V = ti.spec.B, ti.spec.N, ti.spec.V
    n = B * (N + 1)
    zd = np.concatenate([_drafter_rows(ti, 23), np.zeros((3, V), np.float32)])
    rows = np.random.default_rng(29).permutation(n).astype(np.int32).reshape(B, N + 1)
    temps = np.full(n, 0.9, np.float32)                          # per node
    temps[3::7] = 0.0                                            # greedy-drafted nodes
    bad = rows.copy()
    bad[0, 0] = n + 3                                            # tree 0's root: no drafter row
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, path, acc = _run(gpu, ti, zd, 0.9, rows=bad, temps=temps, err=err)
    assert int(err.item()) & gpu.DEVERR_ROW_INDEX
    _check_oracle(ti, zd, 0.9, out, path, acc, rows=bad, temps=temps, skip=(0,))
    # tree 0: its root's q is 0, so every child of the root with p > 0 is accepted
    kids = [i for i in range(1, N + 1) if ti.parents[0, i - 1] == 0]
    if kids:
        assert acc[0] >= 1 and path[0, 0] == kids[0]


def test_tree_lq_ragged_bf16_and_bare_root(gpu):
    spec = TREE_CONFIGS["tree-mid"]
    ti = make_tree_inputs(spec)
    B, N = spec.B, spec.N
    V = 1001
    rng = np.random.default_rng(31)
    z = (3.0 * rng.standard_normal((B, N + 1, V))).astype(np.float32)
    q = np.full((B, N + 1, V), 1.0 / V, np.float32)
    tokens = rng.integers(0, V, size=(B, N)).astype(np.int32)
    ti2 = synth.TreeInputs(spec=synth.TreeSpec(**{**spec.__dict__, "V": V, "dtype": "bf16"}),
                           logits=synth.f32_to_bf16_bits(z), draft_probs=q,
                           parents=ti.parents.copy(), tokens=tokens, uniforms=ti.uniforms)
    parents = ti2.parents.copy()
    # tree 2: node 1 names itself as parent (invalid, absent) and every other
    # node hangs below it, so the root has no child and the token is drawn
    # from the root's p
    parents[2, :] = 1
    zd = _drafter_rows(ti2, 37, scale=0.5)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    out, path, acc = _run(gpu, ti2, zd, 0.8, parents=parents, err=err)
    assert int(err.item()) & gpu.DEVERR_TREE
    _check_oracle(ti2, zd, 0.8, out, path, acc, parents=parents, skip=(2,))
    assert acc[2] == 0 and path[2, 0] == -1


def test_tree_lq_max_nodes_and_empty_batch(gpu):
    """Trees of N = 63 nodes (the limit; random shapes, fp32, V = 1000), each
    node's drafter row gathered through a row index; and B = 0."""
    rng = np.random.default_rng(63)
    B, N, V = 4, 63, 1000
    parents = np.stack([np.array([int(rng.integers(max(0, i - 4), i + 1)) for i in range(N)],
                                 np.int32) for _ in range(B)])
    spec = synth.TreeSpec(name="tree-max", B=B, N=N, V=V, dtype="f32", sigma=2.0, boost="none",
                          temperature=0.9, draft_noise=1.0, draft_temperature=0.9,
                          shape="random", widths=(), seed=63)
    ti = synth.TreeInputs(spec=spec,
                          logits=(2.0 * rng.standard_normal((B, N + 1, V))).astype(np.float32),
                          draft_probs=np.full((B, N + 1, V), 1.0 / V, np.float32),
                          parents=parents, tokens=rng.integers(0, V, size=(B, N)).astype(np.int32),
                          uniforms=rng.random((B, N + 1), dtype=np.float32))
    zd = _drafter_rows(ti, 67, scale=0.3)
    n = B * (N + 1)
    rows = rng.permutation(n).astype(np.int32).reshape(B, N + 1)
    out, path, acc = _run(gpu, ti, zd, 0.9, rows=rows)
    _check_oracle(ti, zd, 0.9, out, path, acc, rows=rows)
    e = torch.zeros((0, N + 1, V), dtype=torch.float32, device=DEV)
    o, p, a = gpu.spec_verify_tree_lq(e, dev(zd), torch.zeros((0, N + 1, 4), dtype=torch.int32,
                                                               device=DEV),
                                      torch.zeros((0, N), dtype=torch.int32, device=DEV),
                                      torch.zeros((0, N), dtype=torch.int32, device=DEV),
                                      torch.zeros((0, N + 1), dtype=torch.float32, device=DEV),
                                      0.9)
    assert o.shape == (0, N + 1) and p.shape == (0, N + 1) and a.shape == (0,)
