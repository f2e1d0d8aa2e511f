"""Oracle DyTC router: EMA acceptance predictor, latency model, draft plan.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What it follows:
  * CAS-Spec blog, section 3.1: accept_rate <- alpha * current_rate +
    (1 - alpha) * accept_rate with alpha = 0.2;
  * CAS-Spec blog, section 3.2: latency = b0 + b1 * seq_len + b2 *
    layer_depth, with b fitted offline;
  * CAS-Spec blog, section 4.1: initial acceptance 0.6-0.7;
  * CAS-Spec abstract: DyTC routes the draft levels and assigns their draft
    lengths from acceptance-rate and latency-prediction heuristics;
  * CAS-Spec blog, section 2.2: three levels, fast L1 .. precise L3.

Readings (listed in the design doc): layer_depth = executed layers; one model is
fitted by least squares over timings of every level (so b2 is identifiable);
the initial acceptance is 0.65; the window is a chain ordered precise level
first; a plan (k per level, total <= K) maximizes (E + 1) / (predicted draft
time + predicted verify time) where E = sum_i prod_{m<=i} a_level(m) is the
expected accepted length; ties go to the smaller total, then larger k of the
most precise level, then the next.  After a round each level that had a
slot at or before the first rejection updates its EMA with its own
accepted / reached ratio.

Tree routing (``plan_tree``, ``update_tree``; the abstract's tree cascade
read as the cascade's levels assigned to the depths of a token tree):
  * a plan is a width B and a length per level; the depths of the tree are
    drafted by the levels in the chain window's order (most precise level
    first), the B first nodes are the first level's B most likely tokens;
  * expected accepted length: the first depth is hit with probability
    1 - (1 - a)^B (each of the B first candidates read as an independent
    try at the level's rate a), each later depth then with its level's rate:
    E = h * (1 + sum_{j>=2} prod_{2<=m<=j} a_level(m)); B = 1 is the chain's E;
  * cost: a pass over r rows costs its level's predicted time times
    row_cost[r - 1] (an input measured on the engine; the latency model of
    section 3.2 prices one row): the first depth's pass has one row (the
    pending token), every later depth's pass B rows, the verify 1 + B D;
  * the plan maximizes (E + 1) / cost over 1 <= B <= b_max and totals
    D <= k_max with B D <= nodes_max; ties go to fewer nodes, then the
    smaller width, then the chain order of ``plan_cascade``;
  * update: the EMA keeps each level's top-1 acceptance: the first depth
    counts as accepted only when the most likely first node (branch 0) is
    the full model's token; later depths count along the branch followed.

Pins (tests/test_oracle_dytc.py): EMA closed form, all-zero acceptance gives
the empty plan, brute enumeration agreement on small cases, least squares on
exactly linear data; tree plans: hand-computed golden cases
(tests/golden/dytc_tree.txt), B = 1 equals the chain router, the expected
length against a Monte Carlo simulation of the acceptance model, the update
against the chain update and hand-computed cases.
"""
import numpy as np

ALPHA = 0.2
A_INIT = 0.65


def ema_update(a, r):
    return ALPHA * r + (1.0 - ALPHA) * a


def predict_latency(beta, seq_len, depth):
    return beta[0] + beta[1] * float(seq_len) + beta[2] * float(depth)


def fit_latency(samples):
    """Least squares b for samples [(seq_len, depth, seconds)]."""
    A = np.array([[1.0, float(s), float(d)] for s, d, _ in samples])
    y = np.array([float(t) for _, _, t in samples])
    beta, *_ = np.linalg.lstsq(A, y, rcond=None)
    return tuple(float(b) for b in beta)


def _window_levels(plan):
    """Level index of every window slot, most precise level first."""
    levels = []
    for lev in reversed(range(len(plan))):
        levels += [lev] * plan[lev]
    return levels


def expected_accepted(a, plan):
    e, prod = 0.0, 1.0
    for lev in _window_levels(plan):
        prod *= a[lev]
        e += prod
    return e


def plan_cost(t_hat, t_verify, plan):
    cost = t_verify
    for lev in reversed(range(len(plan))):
        cost += plan[lev] * t_hat[lev]
    return cost


def plan_cascade(a, t_hat, t_verify, k_max):
    """Draft length per level (index 0 = fastest level), total <= k_max."""
    nl = len(a)
    best, best_key = None, None

    def rec(prefix):
        nonlocal best, best_key
        if len(prefix) == nl:
            plan = list(reversed(prefix))      # prefix was built precise-first
            tot = sum(plan)
            score = (expected_accepted(a, plan) + 1.0) / plan_cost(t_hat, t_verify, plan)
            key = (score, -tot) + tuple(plan[lev] for lev in reversed(range(nl)))
            if best_key is None or key > best_key:
                best, best_key = plan, key
            return
        used = sum(prefix)
        for kk in range(0, k_max - used + 1):
            rec(prefix + [kk])

    rec([])
    return best


def update_cascade(a, slot_levels, n):
    """EMA update after a round with window ``slot_levels`` and n accepted."""
    a = list(a)
    k = len(slot_levels)
    reached = min(n + 1, k)
    for lev in range(len(a)):
        r_cnt = sum(1 for i in range(reached) if slot_levels[i] == lev)
        a_cnt = sum(1 for i in range(n) if slot_levels[i] == lev)
        if r_cnt > 0:
            a[lev] = ema_update(a[lev], a_cnt / r_cnt)
    return a


NODES_MAX = 15


def first_hit(a, B):
    """Probability that one of B independent tries at rate a hits (a itself
    for one try)."""
    return a if B == 1 else 1.0 - (1.0 - a) ** B


def expected_tree(a, B, plan):
    """Expected accepted nodes of a width-B tree whose depths are drafted by
    the levels of ``plan`` in window order (most precise first)."""
    levels = _window_levels(plan)
    if not levels:
        return 0.0
    prod = first_hit(a[levels[0]], B)
    e = prod
    for lev in levels[1:]:
        prod *= a[lev]
        e += prod
    return e


def _rc(row_cost, r):
    return 1.0 if row_cost is None else float(row_cost[r - 1])


def tree_cost(t_hat, t_verify, row_cost, B, plan):
    """Predicted time of a tree round: the depth passes (1 row for the first
    depth, B rows for every later one) and the verify of 1 + B D rows."""
    levels = _window_levels(plan)
    cost = t_verify * _rc(row_cost, 1 + B * len(levels))
    for lev in reversed(range(len(plan))):       # window order, one level at a time
        if plan[lev] == 0:
            continue
        first = 1 if levels[0] == lev else 0     # this level drafts the first depth
        w = first * _rc(row_cost, 1) + (plan[lev] - first) * _rc(row_cost, B)
        cost += w * t_hat[lev]
    return cost


def plan_tree(a, t_hat, t_verify, row_cost, k_max, b_max, nodes_max=NODES_MAX):
    """(B, draft length per level) of the next tree round (index 0 = fastest
    level); a total of 0 is a greedy step (B = 1)."""
    nl = len(a)
    best, best_key = None, None
    for B in range(1, b_max + 1):
        dmax = min(k_max, nodes_max // B)

        def rec(prefix):
            nonlocal best, best_key
            if len(prefix) == nl:
                plan = list(reversed(prefix))
                tot = sum(plan)
                score = (expected_tree(a, B, plan) + 1.0) / tree_cost(t_hat, t_verify, row_cost, B, plan)
                key = (score, -B * tot, -B) + tuple(plan[lev] for lev in reversed(range(nl)))
                if best_key is None or key > best_key:
                    best, best_key = (B, plan), key
                return
            used = sum(prefix)
            for kk in range(0, dmax - used + 1):
                rec(prefix + [kk])

        rec([])
    return best


def update_tree(a, depth_levels, n, branch):
    """EMA update after a tree round: depth_levels[j - 1] drafted depth j, n
    nodes were accepted along branch ``branch`` (-1: none)."""
    a = list(a)
    D = len(depth_levels)
    top1 = n >= 1 and branch == 0
    reached = min(n + 1, D)
    for lev in range(len(a)):
        r_cnt = sum(1 for i in range(reached) if depth_levels[i] == lev)
        a_cnt = sum(1 for i in range(min(n, D)) if depth_levels[i] == lev and (i > 0 or top1))
        if r_cnt > 0:
            a[lev] = ema_update(a[lev], a_cnt / r_cnt)
    return a
