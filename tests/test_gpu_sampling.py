"""GPU parity of speculative sampling on the 4-layer float32 model.

The HIP path draws every random number from the same counter-based streams
as the oracle (``oracle.sampling``), so with float32 logits within 1e-6 of
the oracle's the emitted tokens and the per-round acceptance counts must be
equal, as long as no decision of the oracle run sits within the logits'
error of its threshold (checked on the oracle's recorded margins first).
GPU-only properties: an empty-mask draft (q = p bit for bit) is accepted in
full; runs are reproducible and seed dependent; the first emitted token of a
round is distributed as the GPU's own full-model softmax (chi-square).
"""
import numpy as np
import pytest

import lss_synth
import oracle
from oracle import sampling as smp

pytestmark = pytest.mark.gpu

G = 48
MARGIN = 1e-3        # oracle decisions closer than this to their threshold are not compared

POLICIES = {
    "ar_T1": ({"mode": "ar"}, oracle.Policy(K=0)),
    "static_12_K4_T1": ({"mode": "static", "k_max": 4, "skip": (1, 2)}, oracle.Policy(K=4, skip=(1, 2))),
    "quant_skip1_K4_T07": ({"mode": "static", "k_max": 4, "skip": (1,), "quant": True},
                           oracle.Policy(K=4, skip=(1,), quant=True)),
    "tau_skip2_K5_T07": ({"mode": "static", "k_max": 5, "skip": (2,), "exit_tau": 0.3},
                         oracle.Policy(K=5, skip=(2,), tau=0.3)),
    "dp_S2_I4_T1": ({"mode": "dp", "k_max": 4, "n_skip": 2, "interval": 4},
                    oracle.Policy(K=4, dp_skip=2, interval=4)),
    "cascade_T1": ({"mode": "cascade", "k_max": 8, "interval": 5,
                    "levels": [(3, 1, False), (1, 0, True), (0, 0, True)], "beta": (0.1, 0.0, 0.05)},
                   oracle.Policy(K=8, cascade=[(3, 1, False), (1, 0, True), (0, 0, True)], interval=5,
                                 latency_beta=(0.1, 0.0, 0.05))),
}


@pytest.fixture(scope="module")
def tiny():
    from layer_skip_self_amd import Engine
    shape = lss_synth.SHAPES["tiny"]
    w_cpu = lss_synth.make_weights(shape, device="cpu")
    w_gpu = [(n, t.to("cuda")) for n, t in w_cpu]
    model = oracle.OracleModel(shape, lss_synth.weights_to_numpy(w_cpu))
    prompt = lss_synth.make_prompt(shape, 32)
    eng = Engine(shape, w_gpu, max_seq=256, max_rows=16)
    yield dict(shape=shape, model=model, prompt=prompt, eng=eng)
    eng.set_sampling(0.0)
    eng.close()


def _oracle_run(tiny, pol, T, seed):
    import dataclasses
    sts = []
    if pol.K == 0:
        toks = oracle.ar_generate(tiny["model"], tiny["prompt"], G, max_seq=256, sampling=(T, seed), state_out=sts)
        recs = None
    else:
        p = dataclasses.replace(pol, temperature=T, seed=seed)
        toks, recs = oracle.speculative_generate(tiny["model"], tiny["prompt"], G, p, max_seq=256, state_out=sts)
    return toks, recs, sts[0].margins


@pytest.mark.parametrize("name", sorted(POLICIES))
def test_sampling_matches_oracle(tiny, name):
    gpol, opol = POLICIES[name]
    T = 0.7 if "T07" in name else 1.0
    seed = 1000 + sorted(POLICIES).index(name)
    ref, recs, margins = _oracle_run(tiny, opol, T, seed)
    print(f"{name}: {len(margins)} oracle decisions, smallest margin {min(margins):.3g}", flush=True)
    assert min(margins) > MARGIN, "seed leaves a decision too close to call; pick another"
    toks, st = tiny["eng"].generate(tiny["prompt"], G, dict(gpol, temperature=T, seed=seed))
    assert toks == ref
    if recs is not None:
        assert st["rounds"] == len(recs)
        assert st["accepted"] == sum(r["n"] for r in recs)
        assert st["drafted"] == sum(r["k"] for r in recs)


def test_step_api_matches_oracle(tiny):
    """prefill draw, draft draws, acceptance count and bonus of one round."""
    eng, model, prompt = tiny["eng"], tiny["model"], tiny["prompt"]
    T, seed, mask = 1.0, 4242, [0, 1, 1, 0]
    eng.set_sampling(T, seed)
    t0 = eng.prefill(prompt)
    d = eng.draft(mask, False, 4)
    eng.verify(k=len(d))
    n, b, emitted = eng.accept()
    st, _, _ = oracle.prefill(model, prompt, 256, sampling=(T, seed))
    ot0 = st.t0
    od, _ = oracle.draft(model, st, mask, False, 4, 0.0, (T, seed))
    logits, states, dd = oracle.verify(model, st)
    on, ob, oe = oracle.accept(st, logits, states, dd, (T, seed))
    assert min(st.margins) > MARGIN
    print(f"t0 {t0}, drafts {d}, accepted {n}, bonus {b}")
    assert (t0, d, n, b, emitted) == (ot0, od, on, ob, oe)
    eng.set_sampling(0.0)


def test_error_paths(tiny):
    from layer_skip_self_amd.engine import LssError
    eng = tiny["eng"]
    with pytest.raises(LssError):
        eng.set_sampling(-1.0)
    with pytest.raises(LssError):
        eng.set_sampling(float("nan"))
    eng.set_sampling(1.0, 3)
    eng.prefill(tiny["prompt"])
    with pytest.raises(LssError):              # forced drafts carry no draft distribution
        eng.verify(drafts=[1, 2])
    eng.draft([0, 1, 0, 0], False, 2)
    with pytest.raises(LssError):              # a window is pending
        eng.set_sampling(0.0)
    eng.verify(k=2)
    eng.accept()
    eng.set_sampling(0.0)


def test_sampling_with_w8a8_draft_matches_oracle(tiny):
    """Speculative sampling with a W8A8 draft (q from the int8 draft)."""
    T, seed = 1.0, 1006
    ref, _, margins = _oracle_run(tiny, oracle.Policy(K=4, skip=(1,), quant=2), T, seed)
    print(f"W8A8 + sampling: smallest oracle margin {min(margins):.3g}")
    assert min(margins) > MARGIN, "seed leaves a decision too close to call; pick another"
    tiny["eng"].attach_w8()
    toks, _ = tiny["eng"].generate(tiny["prompt"], G, {"mode": "static", "k_max": 4, "skip": (1,), "quant": 2,
                                                       "temperature": T, "seed": seed})
    assert toks == ref


def test_empty_mask_accepts_every_draft(tiny):
    toks, st = tiny["eng"].generate(tiny["prompt"], G, {"mode": "static", "k_max": 6, "skip": (),
                                                        "temperature": 0.8, "seed": 5})
    assert st["accepted"] == st["drafted"] > 0


def test_reproducible_and_seed_dependent(tiny):
    pol = {"mode": "static", "k_max": 4, "skip": (2,), "temperature": 1.0}
    a, _ = tiny["eng"].generate(tiny["prompt"], G, dict(pol, seed=1))
    b, _ = tiny["eng"].generate(tiny["prompt"], G, dict(pol, seed=1))
    c, _ = tiny["eng"].generate(tiny["prompt"], G, dict(pol, seed=2))
    assert a == b and a != c


def test_first_token_follows_the_full_model_distribution(tiny):
    """Over many seeds, the first token a round emits after a fixed greedy
    prefix is distributed as softmax(z / T) of the GPU's own full-model row
    (the drafts come from a 2-layer-skip draft, so rejections and
    replacement draws both occur)."""
    from scipy import stats
    eng, prompt = tiny["eng"], tiny["prompt"]
    T, mask, N = 1.5, [0, 1, 1, 0], 800
    counts, acc, top, p = None, 0, None, None
    for seed in range(N):
        eng.set_sampling(0.0)
        eng.prefill(prompt)
        eng.set_sampling(T, seed)
        d = eng.draft(mask, False, 1)
        eng.verify(k=len(d))
        if p is None:
            z = eng.read_logits(1)[0].astype(np.float64)
            p = smp.softmax(z, T)
            top = np.argsort(p)[::-1][:6]
            counts = np.zeros(len(top) + 1)
        n, b, emitted = eng.accept()
        acc += n
        hit = np.nonzero(top == emitted[0])[0]
        counts[hit[0] if hit.size else len(top)] += 1
    eng.set_sampling(0.0)
    exp = np.append(p[top], 1 - p[top].sum()) * N
    chi = stats.chisquare(counts, exp)
    print(f"accepted {acc}/{N}; chi-square p {chi.pvalue:.3g}")
    assert 0 < acc < N
    assert chi.pvalue > 1e-4, (counts, exp)


@pytest.mark.parametrize("name", ["ar_T1", "dp_S2_I4_T1"])
def test_sampling_with_stop_token_matches_oracle(tiny, name):
    """A stop token under speculative sampling: the GPU emits the oracle's
    sampled tokens up to and including the stop token's first occurrence
    (the oracle run with the same stop token), and its round count."""
    import dataclasses
    gpol, opol = POLICIES[name]
    T, seed = 1.0, 3000                   # every oracle decision of both runs clears MARGIN at this seed
    full, _, margins = _oracle_run(tiny, opol, T, seed)
    assert min(margins) > MARGIN, "seed leaves a decision too close to call; pick another"
    i = next(j for j in range(6, G) if full[j] not in full[:j])
    stop = (int(full[i]),)
    toks, st = tiny["eng"].generate(tiny["prompt"], G, dict(gpol, temperature=T, seed=seed, stop=stop))
    assert toks == full[:i + 1]
    assert st["emitted"] == i + 1
    if opol.K > 0:
        p = dataclasses.replace(opol, temperature=T, seed=seed, stop=stop)
        ref, recs = oracle.speculative_generate(tiny["model"], tiny["prompt"], G, p, max_seq=256)
        assert ref == toks
        assert st["rounds"] == len(recs)
    else:
        assert oracle.ar_generate(tiny["model"], tiny["prompt"], G, max_seq=256, sampling=(T, seed), stop=stop) == toks
