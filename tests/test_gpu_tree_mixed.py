"""GPU: tree verification of mixed serving batches (spec_verify_tree_mixed and
its early-exit form): tree b walked greedily when temperatures[b] = 0 (or
invalid: flagged) and by rejection sampling at temperatures[b] otherwise.

Every tree against the oracle (greedy trees exactly, sampled ones with the
1e-6 near-tie rule); a batch at one temperature equals spec_verify_tree at
that temperature bit for bit, and an all-greedy batch equals the greedy
call; the early-exit form's greedy trees equal the full call's.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth import TREE_CONFIGS, make_tree_inputs
from tests.gpu_util import DEV, TIE_TOL, dev

pytestmark = pytest.mark.gpu


def _check(ti, temps, out, path, acc, max_flag_frac=0.02):
    flags = 0
    for b in range(ti.spec.B):
        z64 = oracle.decode_logits(ti.logits[b], ti.spec.dtype)
        a = int(acc[b])
        if oracle.mixed.is_greedy(temps[b]):
            wa, wo, wn = oracle.tree.verify_tree_greedy_seq(z64, ti.parents[b], ti.tokens[b])
            assert a == wa and np.array_equal(out[b], wo) and np.array_equal(path[b], wn), b
            continue
        got = (tuple(int(x) for x in path[b, :a]), int(out[b, a]))
        canon, allowed = oracle.tree.tree_outcomes(z64, ti.draft_probs[b], ti.parents[b],
                                                   ti.tokens[b], ti.uniforms[b],
                                                   float(temps[b]), tol=TIE_TOL)
        assert got in allowed, (b, got, canon, allowed)
        flags += got != canon
        assert np.all(out[b, a + 1:] == -1) and np.all(path[b, a:] == -1)
    assert flags <= max(2, max_flag_frac * ti.spec.B)


def _call(sv, fn, ti, temps, err=None):
    r = fn(dev(ti.logits), dev(ti.parents), dev(ti.tokens), dev(temps), dev(ti.draft_probs),
           dev(ti.uniforms), device_error=err)
    torch.cuda.synchronize()
    return [x.cpu().numpy() for x in r]


@pytest.mark.parametrize("name", ["tree-mid", "tree-large"])
def test_mixed_trees_match_oracle(gpu, name):
    ti = make_tree_inputs(TREE_CONFIGS[name])
    B = ti.spec.B
    temps = synth.make_temperatures(B, 61)
    temps[1] = np.nan                                  # invalid: flagged, walked greedily
    assert (temps == 0).any() and (temps > 0).any()
    for fn in (gpu.spec_verify_tree_mixed, gpu.spec_verify_tree_mixed_early_exit):
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        out, path, acc = _call(gpu, fn, ti, temps, err)
        assert int(err.item()) & gpu.DEVERR_TEMPERATURE
        _check(ti, temps, out, path, acc)
    # the early-exit form's greedy trees equal the full call's
    full = _call(gpu, gpu.spec_verify_tree_mixed, ti, temps)
    ee = _call(gpu, gpu.spec_verify_tree_mixed_early_exit, ti, temps)
    for b in range(B):
        if oracle.mixed.is_greedy(temps[b]):
            assert all(np.array_equal(x[b], y[b]) for x, y in zip(full, ee)), b


def test_uniform_batches_equal_the_single_temperature_call(gpu):
    ti = make_tree_inputs(TREE_CONFIGS["tree-mid"])
    B = ti.spec.B
    for T in (0.7, 0.0):
        temps = np.full(B, T, np.float32)
        mixed = _call(gpu, gpu.spec_verify_tree_mixed, ti, temps)
        kw = dict(draft_probs=dev(ti.draft_probs), uniforms=dev(ti.uniforms)) if T > 0 else {}
        one = gpu.spec_verify_tree(dev(ti.logits), dev(ti.parents), dev(ti.tokens), T, **kw)
        torch.cuda.synchronize()
        for x, y in zip(mixed, one):
            assert np.array_equal(x, y.cpu().numpy()), T
