"""The oracle's reading of batch > 1: independent sequences, each decoded
exactly as on its own.  Pins: every sequence of a ragged batch is lossless
(its tokens are its own greedy decoding), a batch of one is the
single-sequence run, and permuting the prompts permutes the results."""
import numpy as np
import pytest

import lss_synth
import oracle

G = 24


@pytest.fixture(scope="module")
def prompts():
    sh = lss_synth.SHAPES["tiny"]
    full = lss_synth.make_prompt(sh, 64)
    rng = np.random.default_rng(5)
    return [full[:32], rng.integers(0, sh.vocab, 20), full[7:52]]


POLICIES = {
    "static": oracle.Policy(K=4, skip=(1, 2)),
    "dp": oracle.Policy(K=4, dp_skip=2, interval=3),
    "exit": oracle.Policy(K=5, skip=(2,), tau=0.3),
}


@pytest.mark.parametrize("name", sorted(POLICIES))
def test_every_sequence_is_its_own_greedy_decoding(tiny_model, prompts, name):
    res = oracle.batch_generate(tiny_model, prompts, G, POLICIES[name])
    assert len(res) == len(prompts)
    for p, (toks, recs) in zip(prompts, res):
        assert toks == oracle.ar_generate(tiny_model, np.asarray(p), G)
        assert all(0 <= r["n"] <= r["k"] for r in recs)


def test_batch_of_one_and_permutation(tiny_model, prompts):
    pol = POLICIES["dp"]
    one = oracle.batch_generate(tiny_model, prompts[:1], G, pol)
    assert one == [oracle.speculative_generate(tiny_model, np.asarray(prompts[0]), G, pol)]
    fwd = oracle.batch_generate(tiny_model, prompts, G, pol)
    rev = oracle.batch_generate(tiny_model, prompts[::-1], G, pol)
    assert fwd == rev[::-1]
