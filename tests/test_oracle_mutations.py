"""Planted mistakes: each mutant of the oracle must fail one of its pins.

A mutant is the oracle's own source with one plausible slip applied (a dropped
term, a wrong sign or index, swapped operands, an off-by-one), compiled on the
CPU into a throwaway namespace.  The real oracle is never modified.
"""
import inspect
import sys
import types

import numpy as np
import pytest

import oracle.peagle as opeagle
import oracle.verify as overify
from tests.pins import blackbox_law, closed_form_law, law_distance, random_case
from tests.test_oracle_build import _case, check_invariants, check_slots_dense


def _mutant_module(mod, func_names, old, new):
    """Copy of ``mod`` recompiled from its source with ``old`` replaced by
    ``new`` inside the functions ``func_names`` (each must contain it), so
    every call inside the copy sees the slip."""
    full = inspect.getsource(mod)
    for name in func_names:
        src = inspect.getsource(getattr(mod, name))
        assert old in src, (name, old)
        assert full.count(src) == 1
        full = full.replace(src, src.replace(old, new))
    m = types.ModuleType(mod.__name__ + "_mutant")
    sys.modules[m.__name__] = m          # dataclasses look their module up
    try:
        exec(compile(full, f"<mutant of {mod.__name__}>", "exec"), m.__dict__)
    finally:
        del sys.modules[m.__name__]
    return m


VERIFY_MUTANTS = [
    ("dropped max(0, .)", ["residual"], "np.maximum(0.0, p - q)", "(p - q)"),
    ("swapped p and q", ["accept_ratio"], "return p_x / q_x", "return q_x / p_x"),
    ("draft tested on the next row", ["verify_sample_seq"],
     "ratio = accept_ratio(p[k][x], q[k, x])", "ratio = accept_ratio(p[min(k + 1, K)][x], q[k, x])"),
    ("bonus from row K-1", ["verify_sample_seq"], "mass, from_p = p[K], True", "mass, from_p = p[K - 1], True"),
    ("temperature dropped", ["target_distribution"], "(z - m) / np.float64(T)", "(z - m)"),
    ("sign of the exponent", ["target_distribution"], "np.exp((z - m) / np.float64(T))",
     "np.exp((m - z) / np.float64(T))"),
    ("residual from the draft side", ["verify_sample_seq"], "mass = residual(p[a], q[a])",
     "mass = residual(q[a], p[a])"),
    ("non-strict accept", ["verify_sample_seq"], "ok = np.float64(u[k]) < ratio",
     "ok = np.float64(u[k]) <= ratio * 0.999"),
]


@pytest.mark.parametrize("label,funcs,old,new", VERIFY_MUTANTS, ids=[m[0] for m in VERIFY_MUTANTS])
def test_verify_mutant_fails_exact_law(label, funcs, old, new):
    m = _mutant_module(overify, funcs, old, new)

    def mutant_ac(z, q, d, u, T):
        tr = m.verify_sample_seq(z, q, d, u, T)
        return tr.a, tr.c

    caught = False
    for seed, (V, K, T) in enumerate([(4, 2, 0.7), (3, 1, 1.0), (5, 2, 1.3)]):
        rng = np.random.default_rng(100 + seed)
        z, q = random_case(rng, V, K, zero_q=(seed == 2))
        try:
            got = blackbox_law(mutant_ac, z, q, T)
            caught |= law_distance(got, closed_form_law(z, q, T)) > 1e-9
        except (AssertionError, IndexError, ValueError):
            caught = True
    assert caught, f"mutant '{label}' passed the exact-law pin"


def test_inverse_cdf_mutant_returns_zero_mass():
    m = _mutant_module(overify, ["inverse_cdf"], "cdf > target", "cdf >= target")
    r = np.array([0.0, 0.5, 0.0, 0.5])
    c, _, _ = m.inverse_cdf(r, 0.0)
    assert r[c] == 0.0            # the strict-comparison pin catches this slip


GREEDY_MUTANTS = [
    ("new token from the next row", "return k, g", "return k, first_argmax(z_rows[min(k + 1, K)])"),
    ("bonus from row K-1", "return K, first_argmax(z_rows[K])", "return K, first_argmax(z_rows[K - 1])"),
]


@pytest.mark.parametrize("label,old,new", GREEDY_MUTANTS, ids=[m[0] for m in GREEDY_MUTANTS])
def test_greedy_mutant_fails_chain_property(label, old, new):
    from tests.test_oracle_greedy import _greedy_chain_property
    m = _mutant_module(overify, ["verify_greedy_seq"], old, new)
    rng = np.random.default_rng(5)
    bad = 0
    for _ in range(200):
        z = rng.standard_normal((4, 5))
        d = [int(x) if rng.random() < 0.6 else int(rng.integers(5)) for x in z[:3].argmax(axis=1)]
        a, c = m.verify_greedy_seq(z, d)
        bad += not _greedy_chain_property(z, d, a, c)
    assert bad > 0, f"mutant '{label}' passed the greedy pin"


BUILD_MUTANTS = [
    ("slot offset off by one", ["slot_of"], "pos % block_size", "(pos + 1) % block_size"),
    ("NTP paired with the previous hidden", ["sequence_rows"], 'rows.append(("ntp", -1, a, a))',
     'rows.append(("ntp", -1, a, max(a - 1, 0)))'),
    ("K MASK rows", ["sequence_rows"], "for m in range(1, K):", "for m in range(0, K):"),
    ("mask position skips one", ["sequence_rows"], 'rows.append(("mask", -1, a + m, -1))',
     'rows.append(("mask", -1, a + m + 1, -1))'),
    ("rejected rows keep their slot", ["build_draft_batch"],
     'slots[row] = (PADDING_SLOT_ID if role == "rejected"', 'slots[row] = (PADDING_SLOT_ID if role == "never"'),
    ("accepted token shifted", ["build_draft_batch"], "ids[row] = int(out_tokens[b, rt])",
     "ids[row] = int(out_tokens[b, rt + 1])"),
]


@pytest.mark.parametrize("label,funcs,old,new", BUILD_MUTANTS, ids=[m[0] for m in BUILD_MUTANTS])
def test_build_mutant_fails_invariants(label, funcs, old, new):
    m = _mutant_module(opeagle, funcs, old, new)
    rng = np.random.default_rng(3)
    K = 5
    case = _case(rng, 12, K, 4, 4)
    with pytest.raises((AssertionError, IndexError)):
        res = m.build_draft_batch(**case)
        check_invariants(res, case, K)
        check_slots_dense(res, case, K)


DRAFT_MUTANTS = [
    ("drafter temperature ignored", ["draft_distribution"], "target_distribution(z, T)",
     "target_distribution(z, 1.0)"),
    ("greedy drafting keeps the last maximum", ["draft_distribution"], "q[first_argmax(z)] = 1.0",
     "q[len(z) - 1 - first_argmax(z[::-1])] = 1.0"),
    ("draw with 1 - u", ["draft_sample_row"], "inverse_cdf(q, float(u))",
     "inverse_cdf(q, 1.0 - float(u))"),
    ("row index transposed", ["_rows"], "np.asarray(row_index, dtype=np.int64).reshape(B, K)",
     "np.asarray(row_index, dtype=np.int64).reshape(K, B).T"),
    ("per-sequence temperatures ignored", ["_temps"], "if temperatures is None:", "if True:"),
    ("default rows shifted by one sequence", ["_rows"],
     "np.arange(B * K, dtype=np.int64).reshape(B, K)",
     "(np.arange(B * K, dtype=np.int64).reshape(B, K) + K) % (B * K)"),
]


@pytest.mark.parametrize("label,funcs,old,new", DRAFT_MUTANTS, ids=[m[0] for m in DRAFT_MUTANTS])
def test_draft_mutant_fails_pins(label, funcs, old, new):
    import oracle.draft as odraft
    from tests.test_oracle_draft import check_module
    m = _mutant_module(odraft, funcs, old, new)
    try:
        fails = check_module(m)
    except (AssertionError, IndexError, ValueError):
        fails = ["raised"]
    assert fails, f"mutant '{label}' passed the drafter pins"


MIXED_MUTANTS = [
    ("first sequence's temperature for all", ["verify_mixed"], "uniforms[b], temperatures[b])",
     "uniforms[b], temperatures[0])"),
    ("NaN temperature sampled", ["is_greedy"], "if not (T32 > 0.0 and np.isfinite(T32)):",
     "if T32 < 0.0:"),
    ("greedy p_draft always 1", ["verify_mixed_seq"],
     "1.0 if int(d[k]) == first_argmax(z_rows[k]) else 0.0", "1.0"),
    ("overflowing log2(e)/T sampled", ["is_greedy"], "return not np.isfinite(c)", "return False"),
    ("reciprocal rule instead of the exponent scale", ["is_greedy"],
     "c = np.float32(LOG2E / np.float64(T32))", "c = np.float32(1.0 / np.float64(T32))"),
]


@pytest.mark.parametrize("label,funcs,old,new", MIXED_MUTANTS, ids=[m[0] for m in MIXED_MUTANTS])
def test_mixed_mutant_fails_pins(label, funcs, old, new):
    import oracle.mixed as omixed
    from tests.test_oracle_mixed import check_module
    m = _mutant_module(omixed, funcs, old, new)
    try:
        fails = check_module(m)
    except (AssertionError, IndexError, ValueError, FloatingPointError):
        fails = ["raised"]
    assert fails, f"mutant '{label}' passed the mixed-batch pins"


METRICS_MUTANTS = [
    ("emitted without the new token", ["counters"], '"emitted": int(a.sum()) + int(a.size)',
     '"emitted": int(a.sum())'),
    ("histogram shifted", ["counters"], "hist[x] += 1", "hist[max(x - 1, 0)] += 1"),
    ("conditional rate over all rounds", ["rates"], "passed / np.maximum(reached, 1)",
     "passed / max(c['rounds'], 1)"),
    ("steps not summed", ["accumulate"], 'for k in ("steps", "rounds"', 'for k in ("rounds"'),
]


@pytest.mark.parametrize("label,funcs,old,new", METRICS_MUTANTS,
                         ids=[m[0] for m in METRICS_MUTANTS])
def test_metrics_mutant_fails_pins(label, funcs, old, new):
    import oracle.metrics as ometrics
    from tests.test_oracle_metrics import check_module
    m = _mutant_module(ometrics, funcs, old, new)
    try:
        fails = check_module(m)
    except (AssertionError, IndexError, KeyError, ValueError):
        fails = ["raised"]
    assert fails, f"mutant '{label}' passed the metrics pins"


TREE_MUTANTS = [
    ("residual not renormalised", ["verify_tree_sample_seq"], "r, mass = res / S, res",
     "r, mass = res, res"),
    ("siblings tested from the last", ["children"],
     "return [i for i in range(1, len(parent) + 1) if int(parent[i - 1]) == n]",
     "return [i for i in range(len(parent), 0, -1) if int(parent[i - 1]) == n]"),
    ("draw from p after rejections", ["verify_tree_sample_seq"],
     "c, _, _ = inverse_cdf(mass, float(u[0]))", "c, _, _ = inverse_cdf(p, float(u[0]))"),
    ("test against p after a rejection", ["verify_tree_sample_seq"], "ratio = r[x] / q[cur, x]",
     "ratio = p[x] / q[cur, x]"),
    ("greedy takes the last matching child", ["verify_tree_greedy_seq"],
     "nxt = next((i for i in children(parent, cur) if int(token[i - 1]) == g), None)",
     "nxt = next((i for i in reversed(children(parent, cur)) if int(token[i - 1]) == g), None)"),
]


@pytest.mark.parametrize("label,funcs,old,new", TREE_MUTANTS, ids=[m[0] for m in TREE_MUTANTS])
def test_tree_mutant_fails_pins(label, funcs, old, new):
    import oracle.tree as otree
    from tests.test_oracle_tree import check_module
    m = _mutant_module(otree, funcs, old, new)
    try:
        fails = check_module(m)
    except (AssertionError, IndexError, KeyError, ValueError, ZeroDivisionError):
        fails = ["raised"]
    assert fails, f"mutant '{label}' passed the tree pins"


OUTCOME_MUTANTS = [
    ("near accept tie only walks on", ["sample_outcomes"],
     "            walk(k + 1)\n            final(k)\n", "            walk(k + 1)\n"),
    ("near accept tie only rejects", ["sample_outcomes"],
     "            walk(k + 1)\n            final(k)\n", "            final(k)\n"),
    ("accept-test flags never counted", ["sample_outcomes"],
     "            flags += 1\n            walk(k + 1)", "            walk(k + 1)"),
    ("draw flags never counted", ["sample_outcomes"],
     "        if len(cands) > 1:\n            flags += 1", "        if False:\n            flags += 1"),
    ("draw band ignored", ["_draw_candidates"], "if tol <= 0.0:", "if True:"),
    ("draw band one-sided", ["_draw_candidates"], "(lo - tol <= target)", "(lo <= target)"),
    ("zero-mass neighbours admitted", ["_draw_candidates"], "ok = (mass > 0.0) & ", "ok = "),
    ("near test on the ratio's reciprocal", ["sample_outcomes"], "abs(uk - ratio) < tol",
     "abs(uk - 1.0 / ratio) < tol"),
]


@pytest.mark.parametrize("label,funcs,old,new", OUTCOME_MUTANTS,
                         ids=[m[0] for m in OUTCOME_MUTANTS])
def test_outcome_mutant_fails_pins(label, funcs, old, new):
    from tests.test_oracle_sample_exact import check_outcomes
    m = _mutant_module(overify, funcs, old, new)
    try:
        fails = check_outcomes(m)
    except (AssertionError, IndexError, ValueError, ZeroDivisionError):
        fails = ["raised"]
    assert fails, f"mutant '{label}' passed the near-tie enumerator pins"
