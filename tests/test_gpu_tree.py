"""GPU parity of token-tree drafting (width B, depth D) on the 4-layer
float32 model, and its losslessness at the 8B shape (in test_gpu_llama3_8b).
Trees whose depths are drafted by different levels (the cascade routed into
the tree) and the tree-cascade generation loop are checked the same way.

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
        eng.generate(prompt, 8, {"mode": "ar", "tree_width": 2})
    with pytest.raises(LssError):
        eng.generate(prompt, 8, {"mode": "cascade", "k_max": 4, "tree_width": 2, "interval": 4,
                                 "levels": [(2, 0, False)], "row_cost": [1.0, -1.0] + [1.0] * 14})
    eng.prefill(prompt)
    with pytest.raises(LssError):
        eng.draft_tree(None, B=2, D=2, levels=[([0, 1, 1, 0], 0), ([0, 1, 1, 0], 3)])   # quant 3
    with pytest.raises(LssError):
        eng.generate(prompt, 8, {"mode": "static", "skip": (1,), "k_max": 1, "tree_width": 4, "tree_depth": 4})


# ---- draft levels per depth, and the cascade routed into the tree

LEVELS = [([0, 0, 1, 0], 1), ([1, 1, 1, 0], 0), ([0, 1, 1, 1], 0)]


def _oracle_tree_rows(model, st, levels, branches):
    """The oracle's draft rows of a tree: whether no row has a near-tie
    (top-B at the root, top-1 along each branch), and each branch's last
    draft row's logits (the pass over depth D - 1)."""
    import copy
    B = len(branches)
    s0 = copy.deepcopy(st)
    z, _ = oracle.forward_row(model, s0, s0.t0, s0.p, "draft", levels[0][0], levels[0][1])
    srt = np.sort(z)[::-1]
    ok = np.min(srt[:B] - srt[1:B + 1]) > 1e-5
    root_valid = list(s0.valid)
    last = []
    for br in branches:
        sb = copy.deepcopy(s0)
        sb.valid = list(root_valid)
        for j in range(1, len(br)):
            zz, _ = oracle.forward_row(model, sb, br[j - 1], sb.p + j, "draft", levels[j][0], levels[j][1])
            s2 = np.sort(zz)[::-1]
            ok = ok and s2[0] - s2[1] > 1e-5
        last.append(zz)
    return ok, np.stack(last)


@pytest.mark.parametrize("levels", [LEVELS, [([1, 0, 0, 0], 0), ([0, 0, 0, 0], 0)],
                                    [([0, 1, 1, 0], 0), ([0, 1, 0, 1], 1), ([1, 0, 1, 0], 0), ([0, 0, 1, 1], 0)]],
                         ids=["three_levels", "layer0_from_depth2", "four_levels"])
def test_mixed_level_tree_matches_oracle(tiny, levels):
    """Branches of a tree drafted by a level per depth, the last draft
    pass's logits, the tree verify's logits and the acceptance, against the
    oracle.  In the second case layer 0 runs from depth 2 only, so the
    pending token's (unwritten) layer-0 key must stay invisible there: the
    depth-2 draft rows' logits would move otherwise."""
    eng, model, prompt = tiny["eng"], tiny["model"], tiny["prompt"]
    B, D = 3, len(levels)
    eng.prefill(prompt)
    branches = eng.draft_tree(None, B=B, D=D, levels=levels)
    zd = eng.read_logits(B)
    st, _, _ = oracle.prefill(model, prompt, 256)
    lv = [(m, bool(q)) for m, q in levels]
    ref = oracle.draft_tree(model, st, None, None, B, D, levels=lv)[0]
    st0, _, _ = oracle.prefill(model, prompt, 256)
    ok, zlast = _oracle_tree_rows(model, st0, lv, ref)
    assert ok
    assert branches == ref
    derr = float(np.max(np.abs(zd - zlast)))
    print(f"last draft pass: max error {derr:.3g}")
    assert derr <= 1e-4
    eng.verify(k=B * D)
    zg = eng.read_logits(1 + B * D)
    logits, states, obr, kv = oracle.verify_tree(model, st)
    assert float(np.max(np.abs(zg - logits))) <= 1e-4
    n, b, emitted = oracle.accept_tree(st, logits, states, obr, kv)
    assert eng.accept() == (n, b, emitted)


def test_one_level_per_depth_is_the_single_mask_tree(tiny):
    eng, prompt = tiny["eng"], tiny["prompt"]
    mask = [0, 1, 1, 0]
    out = []
    for lv in (None, [(mask, 0)] * 3):
        eng.prefill(prompt)
        br = eng.draft_tree(mask, 0, 3, 3) if lv is None else eng.draft_tree(None, B=3, D=3, levels=lv)
        eng.verify(k=9)
        out.append((br, eng.read_logits(10), eng.accept()))
    assert out[0][0] == out[1][0]
    assert np.array_equal(out[0][1], out[1][1])
    assert out[0][2] == out[1][2]


CASCADE = [(3, 1, False), (1, 0, True), (0, 0, True)]


@pytest.mark.parametrize("bmax,beta,steep", [(1, (1.0, 0.0, 1.0), False), (2, (1.0, 0.0, 1.0), False),
                                             (4, (10.0, 0.0, 0.2), False), (4, (0.0, 0.0, 1.0), False),
                                             (4, (10.0, 0.0, 0.2), True)])
def test_tree_cascade_matches_oracle_and_greedy(tiny, bmax, beta, steep):
    """The generation loop with the levels routed into trees: tokens equal
    the greedy run and the oracle's, and so do the rounds, drafted nodes and
    accepted counts (the router's plans and updates agree round for round)."""
    eng = tiny["eng"]
    rc = tuple(float(r) for r in range(1, 17)) if steep else None
    gp = {"mode": "cascade", "k_max": 6, "interval": 5, "levels": CASCADE, "beta": beta, "tree_width": bmax}
    if rc is not None:
        gp["row_cost"] = rc
    toks, st = eng.generate(tiny["prompt"], G, gp)
    ref, recs = oracle.speculative_generate(tiny["model"], tiny["prompt"], G,
                                            oracle.Policy(K=6, cascade=CASCADE, interval=5, tree_width=bmax,
                                                          latency_beta=beta, row_cost=rc))
    wide = sum(1 for r in recs if r["width"] > 1)
    print(f"bmax {bmax} beta {beta} steep {steep}: {st}, {wide} rounds wider than 1")
    assert toks == tiny["ar"]
    assert toks == ref
    assert st["rounds"] == len(recs)
    assert st["accepted"] == sum(r["n"] for r in recs)
    assert st["drafted"] == sum(r["k"] for r in recs)
