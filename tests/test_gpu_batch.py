"""GPU parity of batch > 1 (several independent sequences per pass).

Each sequence of a batch must be decoded exactly as on its own:
- its tokens, rounds and accepted counts equal the oracle's single-sequence
  run (``oracle.batch_generate``);
- and the GPU's own single-sequence run, bit for bit (every batched row is the
  single-sequence row: same kernels, same per-row arithmetic);
- a batched verify's logits equal the single-sequence verify's logits bit for
  bit, also when the batch needs several passes (rows above max_rows, more
  than 16 sequences).
"""
import numpy as np
import pytest

import lss_synth
import oracle

pytestmark = pytest.mark.gpu

G = 40


def _prompts(sh, n, seed=5):
    rng = np.random.default_rng(seed)
    lens = [32, 20, 45, 9, 27, 38, 14, 50, 23, 31, 17, 41, 12, 36, 25, 44, 19, 29][:n]
    return [rng.integers(0, sh.vocab, m).astype(np.int32) for m in lens]


@pytest.fixture(scope="module")
def tiny():
    from layer_skip_self_amd import Engine
    sh = lss_synth.SHAPES["tiny"]
    w_cpu = lss_synth.make_weights(sh, device="cpu")
    w_gpu = [(n, t.to("cuda")) for n, t in w_cpu]
    model = oracle.OracleModel(sh, lss_synth.weights_to_numpy(w_cpu))
    eng = Engine(sh, w_gpu, max_seq=160, max_rows=16, max_seqs=18)
    one = Engine(sh, w_gpu, max_seq=160, max_rows=16)
    yield dict(sh=sh, model=model, eng=eng, one=one)
    eng.close()
    one.close()


POLICIES = {
    "ar": ({"mode": "ar"}, oracle.Policy(K=0)),
    "static_K4": ({"mode": "static", "k_max": 4, "skip": (1, 2)}, oracle.Policy(K=4, skip=(1, 2))),
    "dp_S2_I3": ({"mode": "dp", "k_max": 4, "n_skip": 2, "interval": 3}, oracle.Policy(K=4, dp_skip=2, interval=3)),
    "exit_K5": ({"mode": "static", "k_max": 5, "skip": (2,), "exit_tau": 0.3},
                oracle.Policy(K=5, skip=(2,), tau=0.3)),
    "quant_K4": ({"mode": "static", "k_max": 4, "skip": (1,), "quant": 1}, oracle.Policy(K=4, skip=(1,), quant=1)),
}


@pytest.mark.parametrize("name", sorted(POLICIES))
def test_batch_matches_oracle_and_single_sequence_runs(tiny, name):
    gp, op = POLICIES[name]
    prompts = _prompts(tiny["sh"], 3)
    toks, stats = tiny["eng"].generate_batch(prompts, G, gp)
    ref = oracle.batch_generate(tiny["model"], prompts, G, op)
    for i, p in enumerate(prompts):
        single, sst = tiny["one"].generate(p, G, gp)
        rtoks, recs = ref[i]
        print(f"{name} seq {i}: {stats[i]}")
        assert toks[i] == single, f"sequence {i}: batch != single-sequence run"
        assert toks[i] == rtoks, f"sequence {i}: batch != oracle"
        assert stats[i] == sst
        if name != "ar":
            assert stats[i]["rounds"] == len(recs)
            assert stats[i]["accepted"] == sum(r["n"] for r in recs)


def test_many_sequences_and_passes(tiny):
    """18 sequences (two passes of at most 16 sequences), K = 6 (7 rows per
    sequence: several passes of at most 16 rows)."""
    gp = {"mode": "dp", "k_max": 6, "n_skip": 1, "interval": 4}
    prompts = _prompts(tiny["sh"], 18, seed=9)
    toks, stats = tiny["eng"].generate_batch(prompts, 24, gp)
    for i, p in enumerate(prompts):
        single, sst = tiny["one"].generate(p, 24, gp)
        assert toks[i] == single, i
        assert stats[i] == sst, i


def test_batched_verify_logits_bitwise(tiny):
    """Prefill 4 sequences, draft with per-sequence masks (two share one),
    verify them in one batch (4 + 5 + 3 + 1 rows: one pass), and compare
    every row's logits with the single-sequence engine's verify."""
    eng, one, sh = tiny["eng"], tiny["one"], tiny["sh"]
    prompts = _prompts(sh, 4, seed=13)
    masks = [[0, 1, 1, 0], [0, 0, 1, 0], [0, 1, 1, 0], [1, 1, 1, 1]]
    ks = [3, 4, 2, 0]
    for i, p in enumerate(prompts):
        eng.select(i)
        eng.prefill(p)
    drafted = eng.batch_draft(list(range(4)), masks, ks)
    eng.batch_verify(list(range(4)))
    zb = eng.read_logits(sum(k + 1 for k in ks))
    res = eng.batch_accept(list(range(4)))
    row = 0
    for i, p in enumerate(prompts):
        one.prefill(p)
        d = one.draft(masks[i], 0, ks[i])
        assert d == drafted[i], f"sequence {i}: drafts differ"
        one.verify(k=ks[i])
        z1 = one.read_logits(ks[i] + 1)
        assert np.array_equal(zb[row:row + ks[i] + 1], z1), f"sequence {i}: logits differ"
        assert one.accept() == res[i]
        row += ks[i] + 1


def test_sequences_are_independent_states(tiny):
    """select() keeps every sequence's state: interleaved single-sequence
    rounds on two sequences give each its own greedy decoding."""
    eng, one, sh = tiny["eng"], tiny["one"], tiny["sh"]
    prompts = _prompts(sh, 2, seed=17)
    ref = [one.generate(p, 12, {"mode": "ar"})[0] for p in prompts]
    out = [[], []]
    for i in (0, 1):
        eng.select(i)
        out[i].append(eng.prefill(prompts[i]))
    for _ in range(11):
        for i in (1, 0):
            eng.select(i)
            eng.draft([0, 1, 1, 0], 0, 2)
            eng.verify(k=2)
            _, _, emitted = eng.accept()
            out[i] += emitted
    for i in (0, 1):
        assert out[i][:12] == ref[i]


def test_batch_error_paths(tiny):
    from layer_skip_self_amd.engine import LssError
    eng, sh = tiny["eng"], tiny["sh"]
    prompts = _prompts(sh, 2)
    with pytest.raises(LssError):
        eng.select(18)                                        # out of range
    for i, p in enumerate(prompts):
        eng.select(i)
        eng.prefill(p)
    with pytest.raises(LssError):
        eng.batch_verify([0, 0])                              # duplicate
    with pytest.raises(LssError):
        eng.batch_draft([0, 1], [[0, 1, 1, 0]] * 2, [2, 2], quant=2)   # W8A8 is single-row
    with pytest.raises(LssError):
        eng.batch_accept([0, 1])                              # nothing verified
    with pytest.raises(LssError):
        eng.generate_batch(prompts, 8, {"mode": "static", "k_max": 1, "skip": (1,), "tree_width": 2})
    with pytest.raises(LssError):
        eng.generate_batch(prompts, 8, {"mode": "static", "k_max": 2, "skip": (1,), "temperature": 1.0})
    eng.set_sampling(0.0)


@pytest.fixture(scope="module")
def small():
    from layer_skip_self_amd import Engine
    sh = lss_synth.SHAPES["small_bf16"]
    w = lss_synth.make_weights(sh, device="cuda")
    eng = Engine(sh, w, max_seq=160, max_rows=32, max_seqs=5)
    one = Engine(sh, w, max_seq=160, max_rows=32)
    yield dict(sh=sh, eng=eng, one=one)
    eng.close()
    one.close()


@pytest.mark.parametrize("kernel", ["vector", "mfma", "mfma_verify"])
def test_bf16_batch_equals_single_sequence_runs(small, kernel):
    gp = {"mode": "dp", "k_max": 6, "n_skip": 1, "interval": 3, "decode_kernel": kernel}
    prompts = _prompts(small["sh"], 5, seed=21)
    try:
        toks, stats = small["eng"].generate_batch(prompts, G, gp)
        for i, p in enumerate(prompts):
            single, sst = small["one"].generate(p, G, gp)
            assert toks[i] == single, i
            assert stats[i] == sst, i
        ar, _ = small["eng"].generate_batch(prompts, G, {"mode": "ar", "decode_kernel": kernel})
        assert ar == toks
    finally:
        small["eng"].set_decode_kernel("vector")
        small["one"].set_decode_kernel("vector")


@pytest.mark.parametrize("name", ["ar", "dp_S2_I3"])
def test_batch_stop_tokens_end_each_sequence_on_its_own(tiny, name):
    """A stop token ends every sequence of a batch at its own first
    occurrence: tokens, rounds and accepted counts equal the oracle's
    single-sequence runs with the same stop token, and the GPU's own
    single-sequence runs; sequences that never emit it run to the end."""
    from dataclasses import replace
    gp, op = POLICIES[name]
    prompts = _prompts(tiny["sh"], 3)
    full = oracle.batch_generate(tiny["model"], prompts, G, op)
    t0 = full[0][0]
    stop = (int(next(t0[j] for j in range(6, G) if t0[j] not in t0[:j])),)
    toks, stats = tiny["eng"].generate_batch(prompts, G, dict(gp, stop=stop))
    ref = oracle.batch_generate(tiny["model"], prompts, G, replace(op, stop=stop))
    assert len(toks[0]) < G                                  # sequence 0 stops early
    for i, p in enumerate(prompts):
        rtoks, recs = ref[i]
        single, sst = tiny["one"].generate(p, G, dict(gp, stop=stop))
        assert toks[i] == rtoks == single, i
        assert stats[i] == sst, i
        assert stats[i]["emitted"] == len(rtoks), i
        if name != "ar":
            assert stats[i]["rounds"] == len(recs)
            assert stats[i]["accepted"] == sum(r["n"] for r in recs)
