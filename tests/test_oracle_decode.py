"""Pins of the oracle's draft / verify / accept loop (CPU only).

Properties the pages fix: speculative decoding is lossless (the output equals
the full model's greedy output; CLaSp article sections 三/四, CAS-Spec
abstract), the accepted length lies in [0, k] with the bonus token appended,
a rejected draft is replaced by the full model's prediction and drafting
restarts there (CLaSp article section 三).
"""
import numpy as np
import pytest

import oracle
from oracle.decode import DecodeState

G = 40


@pytest.fixture(scope="module")
def ar_tokens(tiny_model, tiny_prompt):
    return oracle.ar_generate(tiny_model, tiny_prompt, G)


def test_greedy_prefix_property(tiny_model, tiny_prompt, ar_tokens):
    longer = oracle.ar_generate(tiny_model, tiny_prompt, 2 * G)
    assert longer[:G] == ar_tokens


POLICIES = {
    "static_skip_12_K4": oracle.Policy(K=4, skip=(1, 2)),
    "empty_mask_K6": oracle.Policy(K=6, skip=()),
    "all_skipped_K3": oracle.Policy(K=3, skip=(0, 1, 2, 3)),
    "quant_skip_1": oracle.Policy(K=4, skip=(1,), quant=True),
    "tau_0p3": oracle.Policy(K=5, skip=(2,), tau=0.3),
    "clasp_dp_S2_I4": oracle.Policy(K=4, dp_skip=2, interval=4),
    "cascade": oracle.Policy(K=8, cascade=[(3, 1, False), (1, 0, True), (0, 0, True)],
                             interval=5, latency_beta=(0.1, 0.0, 0.05)),
}


@pytest.mark.parametrize("name", sorted(POLICIES))
def test_speculative_equals_greedy(name, tiny_model, tiny_prompt, ar_tokens):
    toks, recs = oracle.speculative_generate(tiny_model, tiny_prompt, G, POLICIES[name])
    assert toks == ar_tokens
    for r in recs:
        assert 0 <= r["n"] <= r["k"]
    # tokens emitted per round = n + 1, summing to G - 1 after t0
    assert sum(r["n"] + 1 for r in recs) == G - 1


def test_empty_mask_draft_is_accepted_in_full(tiny_model, tiny_prompt):
    _, recs = oracle.speculative_generate(tiny_model, tiny_prompt, G, POLICIES["empty_mask_K6"])
    assert all(r["n"] == r["k"] for r in recs)


def test_forced_wrong_draft_rejects_at_that_slot(tiny_model, tiny_prompt, ar_tokens):
    """Drafts equal to the greedy continuation except slot r (wrong token):
    exactly r - 1 tokens are accepted and the output is unchanged."""
    P = len(tiny_prompt)
    st, _, _ = oracle.prefill(tiny_model, tiny_prompt, P + G + 8)
    done = [st.t0]
    for r in range(1, 5):
        k = 4
        truth = ar_tokens[len(done):len(done) + k]
        forced = list(truth)
        forced[r - 1] = (truth[r - 1] + 1) % tiny_model.V
        st.window = forced
        logits, states, d = oracle.verify(tiny_model, st)
        n, bonus, emitted = oracle.accept(st, logits, states, d)
        assert n == r - 1
        assert bonus == truth[r - 1]
        done += emitted
    assert done == ar_tokens[:len(done)]


def test_all_skipped_draft_token_is_head_of_embedding(tiny_shape, tiny_weights_np, tiny_model, tiny_prompt):
    st, _, _ = oracle.prefill(tiny_model, tiny_prompt, 64)
    toks, _ = oracle.draft(tiny_model, st, [1, 1, 1, 1], False, 1)
    e = tiny_weights_np["embed"][st.t0].astype(np.float64)
    z = tiny_weights_np["lm_head"].astype(np.float64) @ (e / np.sqrt(np.mean(e * e) + 1e-5))
    assert toks[0] == int(np.argmax(z))


def test_draft_mask_hides_unwritten_window_slots(tiny_model, tiny_prompt):
    """A layer skipped at window slot 0 but executed at slot 1 attends only to
    the committed prefix and slot 1 (its own KV): same result as a state whose
    slot-0 KV of that layer is garbage."""
    st1, _, _ = oracle.prefill(tiny_model, tiny_prompt, 64)
    st2, _, _ = oracle.prefill(tiny_model, tiny_prompt, 64)
    oracle.draft(tiny_model, st1, [0, 1, 0, 0], False, 1)
    oracle.draft(tiny_model, st2, [0, 1, 0, 0], False, 1)
    p = st2.p
    st2.k[1, p] = 1e3                      # layer 1 never wrote slot 0
    st2.v[1, p] = -1e3
    a, _ = oracle.draft(tiny_model, st1, [0, 0, 0, 0], False, 1)
    b, _ = oracle.draft(tiny_model, st2, [0, 0, 0, 0], False, 1)
    assert a == b
    assert st1.valid[1] == 0b10 and st1.valid[0] == 0b11


def test_exit_threshold_stops_after_low_confidence_token(tiny_model, tiny_prompt):
    st, _, _ = oracle.prefill(tiny_model, tiny_prompt, 64)
    toks, pm = oracle.draft(tiny_model, st, [0, 0, 0, 0], False, 5, tau=0.999)
    assert len(toks) == 1 and pm[0] < 0.999
    st, _, _ = oracle.prefill(tiny_model, tiny_prompt, 64)
    toks, pm = oracle.draft(tiny_model, st, [0, 0, 0, 0], False, 5, tau=0.0)
    assert len(toks) == 5
    for p in pm:
        assert 0.0 < p <= 1.0


def _first_new_token(toks, lo):
    """Index i >= lo of the first token that does not occur in toks[:i]."""
    return next(i for i in range(lo, len(toks)) if toks[i] not in toks[:i])


STOP_POLICIES = {
    "static_skip_12_K4": oracle.Policy(K=4, skip=(1, 2)),
    "clasp_dp_S2_I4": oracle.Policy(K=4, dp_skip=2, interval=4),
    "tree_B3_D2": oracle.Policy(K=4, skip=(1,), tree_width=3, tree_depth=2),
    "cascade": POLICIES["cascade"],
    "cascade_tree": oracle.Policy(K=8, cascade=[(3, 1, False), (1, 0, True), (0, 0, True)], interval=5,
                                  latency_beta=(0.1, 0.0, 0.05), tree_width=2),
}


@pytest.mark.parametrize("name", sorted(STOP_POLICIES))
def test_stop_token_cuts_the_output_after_its_first_occurrence(name, tiny_model, tiny_prompt, ar_tokens):
    """Decoding is deterministic and lossless, so ending it at a stop token
    yields the greedy output up to and including that token's first
    occurrence, for greedy decoding and every draft policy; a stop token
    never emitted changes nothing."""
    from dataclasses import replace
    i = _first_new_token(ar_tokens, 7)
    stop = (int(ar_tokens[i]),)
    assert oracle.ar_generate(tiny_model, tiny_prompt, G, stop=stop) == ar_tokens[:i + 1]
    pol = replace(STOP_POLICIES[name], stop=stop)
    toks, recs = oracle.speculative_generate(tiny_model, tiny_prompt, G, pol)
    assert toks == ar_tokens[:i + 1]
    # the last round is the one that emitted the stop token
    assert sum(r["n"] + 1 for r in recs[:-1]) < i <= sum(r["n"] + 1 for r in recs)
    absent = next(t for t in range(tiny_model.V) if t not in ar_tokens)
    toks, _ = oracle.speculative_generate(tiny_model, tiny_prompt, G, replace(pol, stop=(absent,)))
    assert toks == ar_tokens


def test_stop_token_equal_to_the_first_token(tiny_model, tiny_prompt, ar_tokens):
    stop = (int(ar_tokens[0]),)
    assert oracle.ar_generate(tiny_model, tiny_prompt, G, stop=stop) == ar_tokens[:1]
    toks, recs = oracle.speculative_generate(tiny_model, tiny_prompt, G, oracle.Policy(K=4, skip=(1,), stop=stop))
    assert toks == ar_tokens[:1] and recs == []
