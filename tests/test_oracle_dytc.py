"""Pins of the oracle's DyTC router (CPU only).

CAS-Spec blog, section 3.1 (EMA with alpha = 0.2), section 3.2 (latency
model), section 4.1 (initial acceptance); CAS-Spec abstract (routing and
draft-length assignment from acceptance and latency heuristics).
"""
import itertools
import os

import numpy as np
import pytest

import oracle
from oracle import dytc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_ema_golden():
    a = oracle.A_INIT
    assert a == 0.65
    with open(os.path.join(GOLDEN, "ema.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            r, want = (float(t) for t in line.split(";"))
            a = oracle.ema_update(a, r)
            assert a == pytest.approx(want, abs=1e-15)


def test_ema_closed_form():
    # constant rate r: a_n = r + 0.8^n (a_0 - r)
    for r in (0.0, 0.3, 1.0):
        a = 0.65
        for n in range(1, 30):
            a = oracle.ema_update(a, r)
            assert a == pytest.approx(r + 0.8 ** n * (0.65 - r), abs=1e-12)


def test_zero_acceptance_gives_empty_plan():
    assert oracle.plan_cascade([0.0, 0.0, 0.0], [1.0, 2.0, 3.0], 5.0, 8) == [0, 0, 0]


def test_free_certain_drafts_fill_the_window_with_precise_level():
    # a = 1 everywhere and zero draft cost: score = (K + 1) / t_verify, ties on the
    # total broken toward the most precise level
    assert oracle.plan_cascade([1.0, 1.0, 1.0], [0.0, 0.0, 0.0], 1.0, 8) == [0, 0, 8]


def test_single_level_matches_geometric_series():
    """One usable level (others certain to fail): expected accepted length of k
    drafts at rate a is the geometric sum a (1 - a^k) / (1 - a)."""
    for a, t, tv in [(0.5, 0.3, 1.0), (0.8, 0.5, 1.0), (0.95, 0.1, 1.0), (0.3, 0.6, 1.0)]:
        best_k = max(range(9), key=lambda k: ((a * (1 - a ** k) / (1 - a)) + 1) / (tv + k * t))
        plan = oracle.plan_cascade([0.0, a, 0.0], [9.0, t, 9.0], tv, 8)
        assert plan == [0, best_k, 0]


def test_plan_total_bounded_and_enumerates_165_options():
    n = sum(1 for p in itertools.product(range(9), repeat=3) if sum(p) <= 8)
    assert n == 165
    rng = np.random.default_rng(0)
    for _ in range(20):
        a = list(rng.uniform(0, 1, 3))
        t = list(rng.uniform(0.1, 1, 3))
        plan = oracle.plan_cascade(a, t, 2.0, 8)
        assert sum(plan) <= 8 and min(plan) >= 0


def test_update_counts_reached_slots():
    # window [L3, L3, L2, L1], n = 1: L3 slot 1 accepted, L3 slot 2 reached and rejected
    a = oracle.update_cascade([0.5, 0.5, 0.5], [2, 2, 1, 0], 1)
    assert a[2] == pytest.approx(0.2 * 0.5 + 0.8 * 0.5)
    assert a[1] == 0.5 and a[0] == 0.5
    a = oracle.update_cascade([0.5, 0.5, 0.5], [2, 1, 0], 3)      # all accepted
    assert a == pytest.approx([0.6, 0.6, 0.6])


def test_latency_fit_recovers_linear_model():
    beta = (0.4, 1e-3, 0.05)
    samples = [(s, d, beta[0] + beta[1] * s + beta[2] * d)
               for s in (128, 512, 1024, 2048) for d in (10, 22, 32)]
    got = oracle.fit_latency(samples)
    np.testing.assert_allclose(got, beta, rtol=1e-9, atol=1e-12)
    assert oracle.predict_latency(got, 700, 16) == pytest.approx(0.4 + 0.7 + 0.8)


# ---- tree routing (the levels assigned to the depths of a token tree)

def _golden_tree():
    plans, updates, costs = [], [], []
    with open(os.path.join(GOLDEN, "dytc_tree.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            kind, rest = line.split(" ", 1)
            fields = [t.strip() for t in rest.split(";")]
            if kind == "PLAN":
                a, t, tv, rc, K, bm, B, plan, score = fields
                plans.append(([float(x) for x in a.split()], [float(x) for x in t.split()], float(tv),
                              None if rc == "-" else [float(x) for x in rc.split()], int(K), int(bm), int(B),
                              [int(x) for x in plan.split()], float(score)))
            elif kind == "UPDATE":
                a, lev, n, br, want = fields
                updates.append(([float(x) for x in a.split()], [int(x) for x in lev.split()], int(n), int(br),
                                [float(x) for x in want.split()]))
            else:
                t, tv, rc, B, plan, want = fields
                costs.append(([float(x) for x in t.split()], float(tv), [float(x) for x in rc.split()], int(B),
                              [int(x) for x in plan.split()], float(want)))
    return plans, updates, costs


def test_tree_plan_golden():
    plans, _, costs = _golden_tree()
    assert len(plans) == 4 and len(costs) == 2
    for t, tv, rc, B, plan, want in costs:
        assert dytc.tree_cost(t, tv, rc, B, plan) == pytest.approx(want, rel=1e-12)
    for a, t, tv, rc, K, bm, B, plan, score in plans:
        assert oracle.plan_tree(a, t, tv, rc, K, bm) == (B, plan)
        got = (dytc.expected_tree(a, B, plan) + 1.0) / dytc.tree_cost(t, tv, rc, B, plan)
        assert got == pytest.approx(score, rel=1e-12)


def test_tree_update_golden():
    _, updates, _ = _golden_tree()
    assert len(updates) == 4
    for a, lev, n, br, want in updates:
        assert oracle.update_tree(a, lev, n, br) == pytest.approx(want, abs=1e-15)


def test_width_one_tree_plan_is_the_chain_plan():
    """b_max = 1 and no row costs: the tree router is the chain router (same
    scores, same tie order) on random rates and times."""
    rng = np.random.default_rng(7)
    for _ in range(60):
        nl = int(rng.integers(1, 4))
        a = list(rng.choice([0.0, 0.3, 0.65, 0.9, 1.0], nl)) if rng.random() < 0.3 else list(rng.uniform(0, 1, nl))
        t = list(rng.uniform(0.05, 1.0, nl))
        K = int(rng.integers(0, 9))
        assert oracle.plan_tree(a, t, 1.0, None, K, 1) == (1, oracle.plan_cascade(a, t, 1.0, K))


def test_tree_update_of_the_top_branch_is_the_chain_update():
    rng = np.random.default_rng(8)
    for _ in range(60):
        a = list(rng.uniform(0, 1, 3))
        lev = sorted(rng.integers(0, 3, int(rng.integers(1, 9))), reverse=True)
        n = int(rng.integers(0, len(lev) + 1))
        want = oracle.update_cascade(a, lev, n)
        assert oracle.update_tree(a, lev, n, 0 if n else -1) == want


def test_expected_tree_length_against_simulation():
    """E of a tree against a Monte Carlo run of its acceptance model: B
    independent tries at the first depth's rate, then each later depth
    accepted at its level's rate until the first rejection."""
    rng = np.random.default_rng(11)
    N = 400_000
    for a, B, plan in [([0.3, 0.8], 3, [2, 1]), ([0.5], 4, [3]), ([0.2, 0.5, 0.9], 2, [1, 2, 2]),
                       ([0.7, 0.1], 1, [1, 2])]:
        levels = []
        for lev in reversed(range(len(plan))):
            levels += [lev] * plan[lev]
        hit = (rng.random((N, B)) < a[levels[0]]).any(axis=1)
        alive = hit.copy()
        count = alive.astype(np.int64)
        for lev in levels[1:]:
            alive &= rng.random(N) < a[lev]
            count += alive
        mean, sd = count.mean(), count.std() / np.sqrt(N)
        assert abs(mean - dytc.expected_tree(a, B, plan)) < 5 * sd + 1e-12, (a, B, plan)


def test_tree_plan_limits():
    """Zero rates: a greedy step; certain free drafts: the deepest tree the
    node budget allows at the smallest width (fewer nodes win the tie)."""
    assert oracle.plan_tree([0.0, 0.0], [0.1, 0.2], 1.0, None, 8, 4) == (1, [0, 0])
    assert oracle.plan_tree([1.0, 1.0], [0.0, 0.0], 1.0, None, 8, 4) == (1, [0, 8])
    rng = np.random.default_rng(9)
    for _ in range(40):
        a = list(rng.uniform(0, 1, 3))
        t = list(rng.uniform(0.05, 1.0, 3))
        B, plan = oracle.plan_tree(a, t, 1.0, None, 8, 8)
        assert 1 <= B <= 8 and B * sum(plan) <= 15 and sum(plan) <= 8
