"""Pins of the oracle's tree drafting (CPU only).

Reading of the pages' "dynamic tree cascade" (CAS abs abstract and method
list; CAS blog section 3): a token tree of width B and depth D -- the draft
model's B most likely tokens for the next position, each extended greedily
by the draft to a branch of D tokens, all verified in one pass with a tree
mask (the row of a node sees the committed prefix, the pending token and
its own branch's earlier nodes).  What fixes the expected values:
  * losslessness: the output equals the full model's greedy output for every
    width, depth and policy (the tree only changes how many tokens a round
    emits);
  * depth 1 and width 1 reduce to the one-token chain; width 1 and depth D
    is the chain of D drafts, round for round;
  * every node row of the tree verify equals the full model's last row over
    the whole sequence (prompt, pending token, the branch up to the node)
    recomputed as one causal block: a sibling or another branch leaking into
    the mask, or a wrong position, fails it;
  * acceptance: n is the longest prefix of the branch that starts with the
    full model's token along which every node is the full model's token
    after the previous one; at depth 1, acceptance is monotone in B;
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


@pytest.mark.parametrize("B,D", [(1, 1), (2, 1), (4, 1), (8, 1), (1, 3), (2, 2), (4, 3), (3, 4)])
@pytest.mark.parametrize("kind", ["static", "dp"])
def test_tree_decoding_is_lossless(tiny_model, tiny_prompt, ar, B, D, kind):
    pol = (oracle.Policy(tree_width=B, tree_depth=D, skip=(1, 2)) if kind == "static"
           else oracle.Policy(tree_width=B, tree_depth=D, dp_skip=2, interval=3))
    toks, recs = oracle.speculative_generate(tiny_model, tiny_prompt, G, pol)
    assert toks == ar
    assert all(0 <= r["n"] <= D for r in recs)


def test_width_one_is_the_chain(tiny_model, tiny_prompt):
    for D in (1, 3):
        t1, r1 = oracle.speculative_generate(tiny_model, tiny_prompt, G,
                                             oracle.Policy(tree_width=1, tree_depth=D, skip=(1, 2)))
        tc, rc = oracle.speculative_generate(tiny_model, tiny_prompt, G, oracle.Policy(K=D, skip=(1, 2)))
        assert t1 == tc
        assert [r["n"] for r in r1] == [r["n"] for r in rc]


def _causal_last_row(m, seq):
    H = np.stack([m.embed_row(t) for t in seq])
    for l in range(m.L):
        H = layer_block(m, l, H)
    return m.head(H[-1])


@pytest.mark.parametrize("B,D", [(4, 1), (3, 3)])
def test_node_rows_equal_a_full_causal_recompute(tiny_model, tiny_prompt, B, D):
    m = tiny_model
    st, _, _ = oracle.prefill(m, tiny_prompt, 64)
    t0 = st.t0
    branches, _ = draft_tree(m, st, [0, 1, 1, 0], False, B, D)
    assert len(branches) == B and all(len(br) == D for br in branches)
    logits, _, _, _ = verify_tree(m, st)
    assert np.max(np.abs(_causal_last_row(m, list(tiny_prompt) + [t0]) - logits[0])) < 1e-9
    for b, br in enumerate(branches):
        for j in range(1, D + 1):
            z = _causal_last_row(m, list(tiny_prompt) + [t0] + br[:j])
            assert np.max(np.abs(z - logits[1 + b * D + j - 1])) < 1e-9


def test_draft_branches_follow_the_draft_model(tiny_model, tiny_prompt):
    """Each branch after its first node is the draft's own greedy chain: node
    j + 1 is the argmax of the draft run over prompt + pending token + the
    branch's first j nodes (a plain chain draft from that state)."""
    m = tiny_model
    mask = [0, 1, 1, 0]
    st, _, _ = oracle.prefill(m, tiny_prompt, 64)
    base = copy.deepcopy(st)
    branches, _ = draft_tree(m, st, mask, False, 3, 3)
    for br in branches:
        sc = copy.deepcopy(base)
        sc.window = []
        z, _ = oracle.forward_row(m, sc, sc.t0, sc.p, "draft", mask, False)
        for j in range(1, 3):
            z, _ = oracle.forward_row(m, sc, br[j - 1], sc.p + j, "draft", mask, False)
            assert br[j] == oracle.argmax_first(z)


def test_acceptance_follows_the_greedy_path(tiny_model, tiny_prompt, ar):
    """From states along the greedy path, with the all-skipped draft and with
    an empty mask (the draft is the full model): n equals the number of
    leading nodes of the branch starting with the greedy token that continue
    the greedy output; an empty-mask tree accepts its full depth."""
    m = tiny_model
    for mask, full in (([1, 1, 1, 1], False), ([0, 0, 0, 0], True)):
        for j in range(6):
            st, _, _ = oracle.prefill(m, list(tiny_prompt) + ar[:j], 64)
            branches, _ = draft_tree(m, st, mask, False, 3, 3)
            logits, states, brs, kv = verify_tree(m, st)
            n, bonus, emitted = accept_tree(st, logits, states, brs, kv)
            assert emitted == ar[j + 1:j + 2 + n]
            hit = [br for br in branches if br[0] == ar[j + 1]]
            expect = 0
            if hit:
                while expect < 3 and hit[0][expect] == ar[j + 1 + expect]:
                    expect += 1
            assert n == expect
            if full:
                assert n == 3


def test_acceptance_is_monotone_in_width(tiny_model, tiny_prompt, ar):
    """Depth 1 along the greedy path, all-skipped draft: accepted iff the
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
            logits, states, branches, kv = verify_tree(m, st)
            n, bonus, emitted = accept_tree(st, logits, states, branches, kv)
            a0 = oracle.argmax_first(logits[0])
            assert n == (1 if a0 in [br[0] for br in branches] else 0)
            assert emitted[0] == ar[j + 1]
            ns.append(n)
        assert ns == sorted(ns)
        flips += ns[0] == 0 and ns[-1] == 1
    assert flips > 0


def test_accepted_keys_values_are_the_branch_positions(tiny_model, tiny_prompt, ar):
    """After a depth-3 round the cache at p + 1 .. p + n holds the accepted
    nodes' keys and values, so the next greedy step equals a recompute."""
    m = tiny_model
    st, _, _ = oracle.prefill(m, tiny_prompt, 64)
    draft_tree(m, st, [0, 0, 0, 0], False, 2, 3)
    logits, states, branches, kv = verify_tree(m, st)
    n, bonus, emitted = accept_tree(st, logits, states, branches, kv)
    assert n == 3
    z, _ = oracle.forward_row(m, st, st.t0, st.p, "full")
    ref = _causal_last_row(m, list(tiny_prompt) + ar[:1] + emitted)
    assert np.max(np.abs(z - ref)) < 1e-9


def test_some_run_accepts_deep_in_a_later_branch(tiny_model, tiny_prompt, ar):
    """The skip-{1} draft with width 3 and depth 3 has rounds where a branch
    other than the first is accepted two or more nodes deep, so the move of
    the accepted nodes' keys and values is exercised by the lossless runs."""
    toks, recs = oracle.speculative_generate(tiny_model, tiny_prompt, 48,
                                             oracle.Policy(tree_width=3, tree_depth=3, skip=(1,)))
    assert toks == oracle.ar_generate(tiny_model, tiny_prompt, 48)
    assert any(r.get("branch", -1) >= 1 and r["n"] >= 2 for r in recs)


# ---- the cascade routed into the tree (levels per depth)

CASCADE = [(3, 1, False), (1, 0, True), (0, 0, True)]


def test_mixed_level_branches_are_chain_drafts(tiny_model, tiny_prompt):
    """A tree whose depths are drafted by different levels: branch 0 is the
    chain window drafted one token per level in the same order (the pinned
    chain draft with its per-layer valid bits), and every branch b continues
    from its first node like that chain with the first token forced."""
    m = tiny_model
    lv = [([0, 0, 1, 0], True), ([1, 1, 1, 0], False), ([0, 1, 1, 1], False)]
    st, _, _ = oracle.prefill(m, tiny_prompt, 64)
    base = copy.deepcopy(st)
    branches, _ = draft_tree(m, st, None, None, 3, 3, levels=lv)
    sc = copy.deepcopy(base)
    chain = []
    for mask, q in lv:
        toks, _ = oracle.draft(m, sc, mask, q, 1, 0.0)
        chain += toks
    assert branches[0] == chain
    for br in branches:
        sc = copy.deepcopy(base)
        sc.window = []
        z, _ = oracle.forward_row(m, sc, sc.t0, sc.p, "draft", lv[0][0], lv[0][1])
        for j in range(1, 3):
            z, _ = oracle.forward_row(m, sc, br[j - 1], sc.p + j, "draft", lv[j][0], lv[j][1])
            assert br[j] == oracle.argmax_first(z)
    # one level at every depth is the single-mask tree
    st1 = copy.deepcopy(base)
    st2 = copy.deepcopy(base)
    b1, _ = draft_tree(m, st1, [0, 1, 1, 0], False, 2, 3)
    b2, _ = draft_tree(m, st2, None, None, 2, 3, levels=[([0, 1, 1, 0], False)] * 3)
    assert b1 == b2


def test_mixed_level_visibility_follows_valid_bits(tiny_model, tiny_prompt):
    """Layer 0 runs at depth 1 only: at depth 2 a level that runs layer 0
    must not see the pending token's (never written) layer-0 key there.  The
    node equals a chain draft where the same slots are invisible."""
    m = tiny_model
    lv = [([1, 0, 0, 0], False), ([0, 0, 0, 0], False)]
    st, _, _ = oracle.prefill(m, tiny_prompt, 64)
    branches, _ = draft_tree(m, st, None, None, 1, 2, levels=lv)
    assert st.valid[0] == 0 and st.valid[1] == 1          # the pending token's bits (depth 1 level)
    st2, _, _ = oracle.prefill(m, tiny_prompt, 64)
    t1, _ = oracle.draft(m, st2, lv[0][0], False, 1, 0.0)
    t2, _ = oracle.draft(m, st2, lv[1][0], False, 1, 0.0)
    assert branches[0] == t1 + t2


@pytest.mark.parametrize("bmax", [1, 2, 4])
@pytest.mark.parametrize("beta", [(1.0, 0.0, 1.0), (10.0, 0.0, 0.2)])
def test_tree_cascade_is_lossless(tiny_model, tiny_prompt, ar, bmax, beta):
    pol = oracle.Policy(K=6, cascade=CASCADE, interval=5, tree_width=bmax, latency_beta=beta)
    toks, recs = oracle.speculative_generate(tiny_model, tiny_prompt, G, pol)
    assert toks == ar
    for r in recs:
        assert 1 <= r["width"] <= bmax and r["width"] * len(r["levels"]) <= 15
        assert 0 <= r["n"] <= len(r["levels"])
        assert r["levels"] == sorted(r["levels"], reverse=True)     # precise level first


def test_width_one_tree_cascade_is_the_chain_cascade(tiny_model, tiny_prompt):
    """b_max = 1 and no row costs: the same plans, drafts, acceptances and
    EMA rates as the chain cascade, round for round."""
    for beta in [(1.0, 0.0, 1.0), (10.0, 0.0, 0.2)]:
        tt, rt = oracle.speculative_generate(tiny_model, tiny_prompt, G,
                                             oracle.Policy(K=6, cascade=CASCADE, interval=5, tree_width=1,
                                                           latency_beta=beta))
        tc, rc = oracle.speculative_generate(tiny_model, tiny_prompt, G,
                                             oracle.Policy(K=6, cascade=CASCADE, interval=5, latency_beta=beta))
        assert tt == tc
        assert [r["n"] for r in rt] == [r["n"] for r in rc]
        assert [r["levels"] for r in rt] == [r["levels"] for r in rc]
        assert [r["a"] for r in rt] == [r["a"] for r in rc]


def test_tree_cascade_uses_width_and_row_costs(tiny_model, tiny_prompt, ar):
    """Without row costs the router builds trees wider than 1; steep row
    costs bring it back to width 1."""
    pol = oracle.Policy(K=6, cascade=CASCADE, interval=5, tree_width=4, latency_beta=(10.0, 0.0, 0.2))
    _, recs = oracle.speculative_generate(tiny_model, tiny_prompt, G, pol)
    assert any(r["width"] > 1 for r in recs)
    steep = tuple(float(r) for r in range(1, 17))
    pol = oracle.Policy(K=6, cascade=CASCADE, interval=5, tree_width=4, latency_beta=(10.0, 0.0, 0.2),
                        row_cost=steep)
    toks, recs = oracle.speculative_generate(tiny_model, tiny_prompt, G, pol)
    assert toks == ar
    assert all(r["width"] == 1 for r in recs)
