"""GPU parity of token-tree drafting (width B, depth D) on the 4-layer
float32 model, and its losslessness at the 8B shape (in test_gpu_llama3_8b).

Against the oracle: the emitted tokens, the rounds and accepted counts, the
first round's branches (the draft's top B, each extended greedily) and the
tree verify's logits row by row.  GPU-only: the tree run equals the GPU's
greedy output bit for bit (each node's row of the tree verify is the
greedy step after its branch's earlier nodes, own keys included), also in
runs where a later branch is accepted several nodes deep, so that
branch's keys and values had to be moved to positions p + 1 .. p + n.
"""
import numpy as np
import pytest

import lss_synth
import oracle
from oracle.decode import top_b

pytestmark = pytest.mark.gpu

G = 48


@pytest.fixture(scope="module")
def tiny():
    from layer_skip_self_amd import Engine
    shape = lss_synth.SHAPES["tiny"]
    w_cpu = lss_synth.make_weights(shape, device="cpu")
    w_gpu = [(n, t.to("cuda")) for n, t in w_cpu]
    model = oracle.OracleModel(shape, lss_synth.weights_to_numpy(w_cpu))
    prompt = lss_synth.make_prompt(shape, 32)
    eng = Engine(shape, w_gpu, max_seq=256, max_rows=16)
    ar, _ = eng.generate(prompt, G, {"mode": "ar"})
    yield dict(shape=shape, model=model, prompt=prompt, eng=eng, ar=ar)
    eng.close()


CASES = ([(B, 1, kind) for B in (1, 2, 4, 8) for kind in ("static", "dp")] + [(8, 1, "all_skipped")] +
         [(B, D, kind) for (B, D) in ((1, 4), (2, 3), (3, 3), (4, 2), (2, 7), (5, 3), (3, 5))
          for kind in ("static", "dp", "all_skipped")])


def _policies(B, D, kind):
    if kind == "static":
        return {"mode": "static", "skip": (1, 2)}, oracle.Policy(tree_width=B, tree_depth=D, skip=(1, 2))
    if kind == "dp":
        return ({"mode": "dp", "n_skip": 2, "interval": 3},
                oracle.Policy(tree_width=B, tree_depth=D, dp_skip=2, interval=3))
    return ({"mode": "static", "skip": (0, 1, 2, 3)},
            oracle.Policy(tree_width=B, tree_depth=D, skip=(0, 1, 2, 3)))


@pytest.mark.parametrize("B,D,kind", CASES)
def test_tree_matches_oracle_and_greedy(tiny, B, D, kind):
    eng = tiny["eng"]
    gp, op = _policies(B, D, kind)
    toks, st = eng.generate(tiny["prompt"], G, dict(gp, tree_width=B, tree_depth=D, k_max=1))
    ref, recs = oracle.speculative_generate(tiny["model"], tiny["prompt"], G, op)
    deep = sum(1 for r in recs if r.get("branch", -1) >= 1 and r["n"] >= 2)
    print(f"B={B} D={D} {kind}: {st['rounds']} rounds, {st['accepted']} accepted, "
          f"{deep} rounds accept a later branch >= 2 deep")
    assert toks == tiny["ar"]
    assert toks == ref
    assert st["rounds"] == len(recs)
    assert st["accepted"] == sum(r["n"] for r in recs)


def test_some_run_accepts_a_later_candidate(tiny):
    """The all-skipped width-8 run accepts candidates past the first, and the
    width-3 depth-3 static run accepts later branches several nodes deep, so
    the key/value moves are exercised by the test above."""
    _, recs = oracle.speculative_generate(tiny["model"], tiny["prompt"], G,
                                          oracle.Policy(tree_width=8, skip=(0, 1, 2, 3)))
    assert any(r.get("branch", -1) >= 1 for r in recs)
    _, recs = oracle.speculative_generate(tiny["model"], tiny["prompt"], G,
                                          oracle.Policy(tree_width=3, tree_depth=3, skip=(1, 2)))
    assert any(r.get("branch", -1) >= 1 and r["n"] >= 2 for r in recs)


@pytest.mark.parametrize("quant", [1, 2])
def test_quantized_tree_drafts_are_lossless(tiny, quant):
    """Int8-activation and W8A8 tree drafts (the latter one branch per pass)
    keep the greedy output."""
    eng = tiny["eng"]
    if quant == 2:
        eng.attach_w8()
    for B, D in ((3, 3), (2, 5)):
        toks, st = eng.generate(tiny["prompt"], G, {"mode": "static", "skip": (1, 2), "k_max": 1, "quant": quant,
                                                    "tree_width": B, "tree_depth": D})
        print(f"quant {quant} B={B} D={D}: {st['rounds']} rounds, {st['accepted']} accepted")
        assert toks == tiny["ar"]
        assert st["accepted"] > 0


def test_branches_and_tree_verify_match_oracle(tiny):
    """First round of a width-3 depth-3 tree: the GPU's branches are the
    oracle's (no near-tie in any draft row), and every row of the tree
    verify matches the oracle's row (pending token, then each branch's
    nodes) within the float32 tolerance of the other tiny-model tests."""
    import copy
    eng, model, prompt = tiny["eng"], tiny["model"], tiny["prompt"]
    mask, B, D = [0, 1, 1, 0], 3, 3
    eng.prefill(prompt)
    branches = eng.draft_tree(mask, 0, B, D)
    st, _, _ = oracle.prefill(model, prompt, 256)
    # the draft's own rows: top-B gaps at the root, top-1 gaps along each branch
    s0 = copy.deepcopy(st)
    z, _ = oracle.forward_row(model, s0, s0.t0, s0.p, "draft", mask, False)
    srt = np.sort(z)[::-1]
    assert np.min(srt[:B] - srt[1:B + 1]) > 1e-5
    ref = oracle.draft_tree(model, st, mask, False, B, D)[0]
    for br in ref:
        sb = copy.deepcopy(s0)
        for j in range(1, D):
            zz, _ = oracle.forward_row(model, sb, br[j - 1], sb.p + j, "draft", mask, False)
            s2 = np.sort(zz)[::-1]
            assert s2[0] - s2[1] > 1e-5, "near-tie in a branch row"
    assert branches == ref
    eng.verify(k=B * D)
    zg = eng.read_logits(1 + B * D)
    logits, states, obr, kv = oracle.verify_tree(model, st)
    err = float(np.max(np.abs(zg - logits)))
    assert err <= 1e-4, err
    got = eng.accept()
    n, b, emitted = oracle.accept_tree(st, logits, states, obr, kv)
    assert got == (n, b, emitted)


def test_candidates_are_the_draft_top_b(tiny):
    eng, model, prompt = tiny["eng"], tiny["model"], tiny["prompt"]
    mask = [0, 1, 1, 0]
    eng.prefill(prompt)
    cands = [br[0] for br in eng.draft_tree(mask, 0, 8)]
    st, _, _ = oracle.prefill(model, prompt, 256)
    z, _ = oracle.forward_row(model, st, st.t0, st.p, "draft", mask, False)
    srt = np.sort(z)[::-1]
    assert np.min(srt[:8] - srt[1:9]) > 1e-5, "near-tie among the top 9"
    assert cands == top_b(z, 8)
    eng.verify(k=8)
    eng.accept()


def test_tree_error_paths(tiny):
    from layer_skip_self_amd.engine import LssError
    eng, prompt = tiny["eng"], tiny["prompt"]
    eng.prefill(prompt)
    with pytest.raises(LssError):
        eng.draft_tree([0, 1, 1, 0], 0, 9)              # B > 8
    with pytest.raises(LssError):
        eng.draft_tree([0, 1, 1, 0], 0, 4, 4)           # 16 nodes > LSS_TREE_NODES_MAX
    with pytest.raises(LssError):
        eng.draft_tree([0, 1, 1, 0], 0, 2, 0)           # depth 0
    eng.set_sampling(1.0, 1)
    with pytest.raises(LssError):
        eng.draft_tree([0, 1, 1, 0], 0, 2)              # greedy only
    eng.set_sampling(0.0)
    cands = [br[0] for br in eng.draft_tree([0, 1, 1, 0], 0, 2)]
    with pytest.raises(LssError):
        eng.draft([0, 1, 1, 0], 0, 1)                   # a tree window is pending
    with pytest.raises(LssError):
        eng.verify(drafts=[1, 2])
    # the rejected call left the candidates in place: the tree round still
    # verifies what draft_tree returned, as the oracle's round does
    eng.verify(k=2)
    got = eng.accept()
    st, _, _ = oracle.prefill(tiny["model"], prompt, 256)
    assert [br[0] for br in oracle.draft_tree(tiny["model"], st, [0, 1, 1, 0], False, 2)[0]] == cands
    logits, states, oc, kv = oracle.verify_tree(tiny["model"], st)
    n, b, emitted = oracle.accept_tree(st, logits, states, oc, kv)
    assert got == (n, b, emitted)
    with pytest.raises(LssError):
        eng.generate(prompt, 8, {"mode": "cascade", "k_max": 4, "tree_width": 2, "interval": 4,
                                 "levels": [(2, 0, False)]})
    with pytest.raises(LssError):
        eng.generate(prompt, 8, {"mode": "static", "skip": (1,), "k_max": 1, "tree_width": 4, "tree_depth": 4})
