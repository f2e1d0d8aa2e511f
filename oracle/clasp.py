"""Oracle CLaSp layer selection: the approximate DP and brute force.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What it follows (CLaSp article):
  * section 二: after verification, the full hidden states of the last
    accepted token are the target for choosing the next draft's skipped
    layers;
  * section 三: the DP's state (i, j) is the best (largest) cosine similarity
    to the optimal hidden state reachable after the first i layers with j of
    them skipped, kept in a state matrix; the recurrence is approximate
    (no strict optimal substructure) but lands close to brute force and far
    above random choice; state (i, j) needs only states (i-1, .), so all j of
    one i can run together, each row seeing the shared prefix plus its own
    key/value (a special mask instead of copying the KV cache).

Readings (listed in the design doc): states are the raw (pre-norm) residual
stream; the similarity at stage i is taken against the target's residual
after layer i-1; exactly S layers end up skipped (j is bounded by lo/hi so
that S stays reachable); the first and last layers may be skipped; a tie
between skip and execute keeps the layer executed; the DP state rows are
forwarded at the target's position t* over the committed prefix [0, t*).

Pins (tests/test_oracle_clasp.py): DP score <= brute-force optimum (and
equality on the tiny model), the recomputed masked forward reproduces the
DP's final state, planted identity layers are recovered exactly, S = 0 and
S = L closed forms.
"""
import itertools

import numpy as np

from .decode import layer_row


def _cos(x, y):
    return float(np.dot(x, y) / (np.linalg.norm(x) * np.linalg.norm(y)))


def clasp_dp(model, st, S, n_layers=None):
    """Choose S layers to skip among the first ``n_layers`` (default all).

    Returns (mask [L] with 1 = skip, score = cos(g[n][S], H*[n]), decisions)
    where ``decisions[(i, j)] = (skip_chosen, cos_skip, cos_exec)`` and layers
    >= n_layers are marked skipped (an early exit).
    """
    L = model.L
    Le = L if n_layers is None else n_layers
    assert 0 <= S <= Le
    H = st.target_states
    tstar = st.target_pos

    def lo(i):
        return max(0, S - (Le - i))

    def hi(i):
        return min(i, S)

    g = {(0, 0): H[0]}
    dec = {}
    for i in range(1, Le + 1):
        for j in range(lo(i), hi(i) + 1):
            exec_ok = lo(i - 1) <= j <= hi(i - 1)
            skip_ok = j >= 1 and lo(i - 1) <= j - 1 <= hi(i - 1)
            ce = cs = None
            if exec_ok:
                xe = layer_row(model, i - 1, g[(i - 1, j)], tstar, st, "dp")
                ce = _cos(xe, H[i])
            if skip_ok:
                xs = g[(i - 1, j - 1)]
                cs = _cos(xs, H[i])
            take_skip = skip_ok and (not exec_ok or cs > ce)
            g[(i, j)] = xs if take_skip else xe
            dec[(i, j)] = (take_skip, cs, ce)
    mask = [0] * L
    j = S
    for i in range(Le, 0, -1):
        if dec[(i, j)][0]:
            mask[i - 1] = 1
            j -= 1
    assert j == 0
    for l in range(Le, L):
        mask[l] = 1
    return mask, _cos(g[(Le, S)], H[Le]), dec


def forward_with_mask_at_target(model, st, mask, n_layers=None):
    """Residual of the target row after ``n_layers`` layers with ``mask``."""
    Le = model.L if n_layers is None else n_layers
    h = st.target_states[0]
    for l in range(Le):
        if not mask[l]:
            h = layer_row(model, l, h, st.target_pos, st, "dp")
    return h


def brute_force_skip(model, st, S, n_layers=None):
    """Best S-subset by exhaustive search (ties -> lexicographically first).

    Returns (mask, score, all scores by subset).
    """
    L = model.L
    Le = L if n_layers is None else n_layers
    H = st.target_states
    best, scores = None, {}
    for combo in itertools.combinations(range(Le), S):
        mask = [1 if l in combo else 0 for l in range(L)]
        c = _cos(forward_with_mask_at_target(model, st, mask, Le), H[Le])
        scores[combo] = c
        if best is None or c > best[1]:
            best = (combo, c)
    mask = [1 if l in best[0] else 0 for l in range(L)]
    for l in range(Le, L):
        mask[l] = 1
    return mask, best[1], scores
