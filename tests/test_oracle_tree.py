"""Pins of the oracle's tree drafting (CPU only).

Reading of the pages' "dynamic tree cascade" (CAS abs abstract and method
list; CAS blog section 3): a token tree, here of width B and depth 1 -- the
draft model's B most likely tokens for the next position, verified in one
pass with a tree mask (each candidate sees the committed prefix, the pending
token and itself).  What fixes the expected values:
  * losslessness: the output equals the full model's greedy output for every
    width and policy (the tree only changes how many tokens a round emits);
  * B = 1 is the chain with one draft token, round for round;
  * a candidate row of the tree verify equals the full model's last row over
    the whole sequence recomputed as one causal block (a sibling leaking into
    the mask, or a wrong position, fails it);
  * from one state, acceptance is monotone in B (accepted iff the greedy
    token is among the draft's top B);
  * top-B ordering with ties to the lowest index.
"""
import copy

import numpy as np
import pytest

import oracle
from oracle.decode import top_b, draft_tree, verify_tree, accept_tree, layer_block

G = 40


def test_top_b_order_and_ties():
    z = np.array([1.0, 3.0, 3.0, 2.0, 5.0, 3.0])
    assert top_b(z, 1) == [4] == [oracle.argmax_first(z)]
    assert top_b(z, 4) == [4, 1, 2, 5]
    assert top_b(z, 6) == [4, 1, 2, 5, 3, 0]


@pytest.fixture(scope="module")
def ar(tiny_model, tiny_prompt):
    return oracle.ar_generate(tiny_model, tiny_prompt, G)


@pytest.mark.parametrize("B", [1, 2, 4, 8])
@pytest.mark.parametrize("kind", ["static", "dp"])
def test_tree_decoding_is_lossless(tiny_model, tiny_prompt, ar, B, kind):
    pol = (oracle.Policy(tree_width=B, skip=(1, 2)) if kind == "static"
           else oracle.Policy(tree_width=B, dp_skip=2, interval=3))
    toks, recs = oracle.speculative_generate(tiny_model, tiny_prompt, G, pol)
    assert toks == ar
    assert all(r["n"] in (0, 1) for r in recs)


def test_width_one_is_the_one_token_chain(tiny_model, tiny_prompt):
    t1, r1 = oracle.speculative_generate(tiny_model, tiny_prompt, G, oracle.Policy(tree_width=1, skip=(1, 2)))
    tc, rc = oracle.speculative_generate(tiny_model, tiny_prompt, G, oracle.Policy(K=1, skip=(1, 2)))
    assert t1 == tc
    assert [r["n"] for r in r1] == [r["n"] for r in rc]


def test_candidate_rows_equal_a_full_causal_recompute(tiny_model, tiny_prompt):
    m = tiny_model
    st, _, _ = oracle.prefill(m, tiny_prompt, 64)
    t0 = st.t0
    cands, _ = draft_tree(m, st, [0, 1, 1, 0], False, 4)
    logits, _, _, _ = verify_tree(m, st)
    for i, c in enumerate(cands):
        seq = list(tiny_prompt) + [t0, c]
        H = np.stack([m.embed_row(t) for t in seq])
        for l in range(m.L):
            H = layer_block(m, l, H)
        z = m.head(H[-1])
        assert np.max(np.abs(z - logits[i + 1])) < 1e-9
    H = np.stack([m.embed_row(t) for t in list(tiny_prompt) + [t0]])
    for l in range(m.L):
        H = layer_block(m, l, H)
    assert np.max(np.abs(m.head(H[-1]) - logits[0])) < 1e-9


def test_acceptance_is_monotone_in_width(tiny_model, tiny_prompt, ar):
    """Along the greedy path, with the all-skipped draft: accepted iff the
    greedy token is among the draft's top B, hence monotone in B; some state
    must reject at B = 1 and accept at a larger width (else the test proves
    nothing)."""
    m = tiny_model
    flips = 0
    for j in range(8):
        base, _, _ = oracle.prefill(m, list(tiny_prompt) + ar[:j], 64)
        ns = []
        for B in range(1, 9):
            st = copy.deepcopy(base)
            draft_tree(m, st, [1, 1, 1, 1], False, B)
            logits, states, cands, kv = verify_tree(m, st)
            n, bonus, emitted = accept_tree(st, logits, states, cands, kv)
            a0 = oracle.argmax_first(logits[0])
            assert n == (1 if a0 in cands else 0)
            assert emitted[0] == ar[j + 1]
            ns.append(n)
        assert ns == sorted(ns)
        flips += ns[0] == 0 and ns[-1] == 1
    assert flips > 0
