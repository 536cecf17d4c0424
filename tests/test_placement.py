"""The offline placement solver (activation_sparse_amd.placement), on the CPU: the exact optimum
of the integer program by brute force on tiny instances, the greedy bound with unequal neuron
sizes, the constraints, and agreement with the fixed top-share rule on one layer."""
import itertools
import math

import numpy as np
import pytest

import synth
from activation_sparse_amd.placement import solve_placement, gpu_impact_share


def _brute(counts, sizes, budget, min_frac):
    """The optimum of the program over every subset (tiny instances)."""
    flat = [(l, i) for l in range(len(counts)) for i in range(len(counts[l]))]
    best = -1
    for mask in itertools.product((0, 1), repeat=len(flat)):
        used = sum(sizes[l] for (l, _), m in zip(flat, mask) if m)
        if used > budget:
            continue
        per = [0] * len(counts)
        for (l, _), m in zip(flat, mask):
            per[l] += m
        if any(per[l] < math.ceil(min_frac * len(counts[l])) for l in range(len(counts))):
            continue
        best = max(best, sum(int(counts[l][i]) for (l, i), m in zip(flat, mask) if m))
    return best


def _value(counts, tables):
    return sum(int(np.sum(np.asarray(c)[t])) for c, t in zip(counts, tables))


def _check_tables(counts, sizes, budget, min_frac, tables):
    assert sum(sizes[l] * len(t) for l, t in enumerate(tables)) <= budget
    for l, t in enumerate(tables):
        assert len(t) >= math.ceil(min_frac * len(counts[l]))
        assert np.all(np.diff(t) > 0) and (len(t) == 0 or (t[0] >= 0 and t[-1] < len(counts[l])))


@pytest.mark.parametrize("seed", range(12))
def test_equal_sizes_reach_the_exact_optimum(seed):
    g = np.random.default_rng(seed)
    L = int(g.integers(2, 4))
    counts = [g.integers(0, 9, size=int(g.integers(2, 6))) for _ in range(L)]
    sizes = [7] * L
    n = sum(len(c) for c in counts)
    budget = 7 * int(g.integers(1, n + 1))
    min_frac = float(g.choice([0.0, 0.2, 0.4]))
    if sum(math.ceil(min_frac * len(c)) for c in counts) * 7 > budget:
        with pytest.raises(ValueError):
            solve_placement(counts, sizes, budget, min_frac)
        return
    tables = solve_placement(counts, sizes, budget, min_frac)
    _check_tables(counts, sizes, budget, min_frac, tables)
    assert _value(counts, tables) == _brute(counts, sizes, budget, min_frac)


@pytest.mark.parametrize("seed", range(12))
def test_unequal_sizes_are_within_one_neuron_of_the_optimum(seed):
    g = np.random.default_rng(100 + seed)
    L = int(g.integers(2, 4))
    counts = [g.integers(0, 9, size=int(g.integers(2, 6))) for _ in range(L)]
    sizes = [int(v) for v in g.integers(3, 12, size=L)]
    budget = int(g.integers(5, 40))
    tables = solve_placement(counts, sizes, budget, 0.0)
    _check_tables(counts, sizes, budget, 0.0, tables)
    best = _brute(counts, sizes, budget, 0.0)
    got = _value(counts, tables)
    assert got <= best and best - got <= max(int(np.max(c)) for c in counts)


def test_one_layer_is_the_fixed_top_share_rule():
    """One layer and a budget of floor(0.4 N) neurons: the tables synth's fixed rule builds
    (count descending, ties to the lower id)."""
    cfg = synth.CONFIGS["opt-30b"]
    spec = synth.layer_spec(cfg, 2)
    n_g = int(math.floor(cfg.gpu_frac * cfg.N))
    t = solve_placement([spec.counts], [1], n_g)[0]
    assert np.array_equal(t, spec.T_g)


def test_budget_moves_to_the_layers_with_more_concentrated_activations():
    """Two layers of the same size, one with a steeper hotness than the other: a shared budget
    favours the steeper one, and the GPU's expected share of all activations is at least the
    per-layer rule's."""
    N = 1000
    rank = np.arange(1, N + 1, dtype=np.float64)
    p = [np.minimum(0.95, 2.0 * rank ** -0.6), np.minimum(0.95, 30.0 * rank ** -1.3)]
    counts = [np.round(256 * q).astype(np.int64) for q in p]
    tables = solve_placement(counts, [1, 1], 800)
    fixed = [np.sort(np.lexsort((np.arange(N), -c))[:400]).astype(np.int32) for c in counts]
    assert len(tables[0]) != len(tables[1])
    assert gpu_impact_share(p, tables) >= gpu_impact_share(p, fixed)


def test_bad_arguments():
    with pytest.raises(ValueError):
        solve_placement([np.ones(4)], [1, 2], 4)
    with pytest.raises(ValueError):
        solve_placement([np.ones(4)], [0], 4)
    with pytest.raises(ValueError):
        solve_placement([np.ones(4)], [1], 4, min_frac=1.5)


def test_solver_tables_of_the_small_gated_stack():
    """The stack the GPU test runs: the solver moves budget between its layers (n_g differs from
    layer to layer), spends all of it, and each table is a valid partition with its complement."""
    from tests.placement_cases import SMALL, solver_specs
    specs = solver_specs(SMALL)
    n_g = [specs[l].n_g for l in range(SMALL.n_layers)]
    k = int(math.floor(SMALL.gpu_frac * SMALL.N))
    assert sum(n_g) == k * SMALL.n_layers
    assert len(set(n_g)) > 1 and max(n_g) - min(n_g) > 64
    for s in specs.values():
        both = np.concatenate([s.T_g, s.T_c])
        assert np.array_equal(np.sort(both), np.arange(SMALL.N))
        assert np.all(np.diff(s.T_g) > 0) and np.all(np.diff(s.T_c) > 0)
        # the solver keeps the hottest neurons: every GPU neuron's count >= every CPU neuron's
        if s.n_g and len(s.T_c):
            assert s.counts[s.T_g].min() >= s.counts[s.T_c].max()


def test_with_table_rejects_bad_ids():
    spec = synth.layer_spec(synth.CONFIGS["opt-768"], 0)
    with pytest.raises(ValueError):
        synth.with_table(spec, np.array([3, 3], np.int32))
    with pytest.raises(ValueError):
        synth.with_table(spec, np.array([spec.cfg.N], np.int32))
