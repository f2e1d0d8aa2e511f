"""GPU parity of width-B token-tree drafting on the 4-layer float32 model,
and its losslessness at the 8B shape (in test_gpu_llama3_8b).

Against the oracle: the emitted tokens, the rounds and accepted counts, and
the first round's candidates (the draft's top B).  GPU-only: the tree run
equals the GPU's greedy output bit for bit (each candidate row of the tree
verify is the greedy step after it, own key included), also in runs where a
candidate other than the first is accepted, so the accepted candidate's
keys and values had to be moved to position p + 1.
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


CASES = [(B, kind) for B in (1, 2, 4, 8) for kind in ("static", "dp")] + [(8, "all_skipped")]


@pytest.mark.parametrize("B,kind", CASES)
def test_tree_matches_oracle_and_greedy(tiny, B, kind):
    eng = tiny["eng"]
    if kind == "static":
        gp, op = {"mode": "static", "skip": (1, 2)}, oracle.Policy(tree_width=B, skip=(1, 2))
    elif kind == "dp":
        gp, op = {"mode": "dp", "n_skip": 2, "interval": 3}, oracle.Policy(tree_width=B, dp_skip=2, interval=3)
    else:
        gp, op = {"mode": "static", "skip": (0, 1, 2, 3)}, oracle.Policy(tree_width=B, skip=(0, 1, 2, 3))
    toks, st = eng.generate(tiny["prompt"], G, dict(gp, tree_width=B, k_max=1))
    ref, recs = oracle.speculative_generate(tiny["model"], tiny["prompt"], G, op)
    rows = [r.get("row", 0) for r in recs]
    print(f"B={B} {kind}: {st['rounds']} rounds, {st['accepted']} accepted, accepted rows {sorted(set(rows))}")
    assert toks == tiny["ar"]
    assert toks == ref
    assert st["rounds"] == len(recs)
    assert st["accepted"] == sum(r["n"] for r in recs)


def test_some_run_accepts_a_later_candidate(tiny):
    """The all-skipped width-8 run accepts candidates past the first, so the
    key/value move of the accepted candidate is exercised by the test above."""
    _, recs = oracle.speculative_generate(tiny["model"], tiny["prompt"], G,
                                          oracle.Policy(tree_width=8, skip=(0, 1, 2, 3)))
    assert any(r.get("row", 0) >= 2 for r in recs)


def test_candidates_are_the_draft_top_b(tiny):
    eng, model, prompt = tiny["eng"], tiny["model"], tiny["prompt"]
    mask = [0, 1, 1, 0]
    eng.prefill(prompt)
    cands = eng.draft_tree(mask, 0, 8)
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
    eng.set_sampling(1.0, 1)
    with pytest.raises(LssError):
        eng.draft_tree([0, 1, 1, 0], 0, 2)              # greedy only
    eng.set_sampling(0.0)
    cands = eng.draft_tree([0, 1, 1, 0], 0, 2)
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
