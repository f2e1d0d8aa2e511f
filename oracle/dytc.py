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

Pins (tests/test_oracle_dytc.py): EMA closed form, all-zero acceptance gives
the empty plan, brute enumeration agreement on small cases, least squares on
exactly linear data.
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
