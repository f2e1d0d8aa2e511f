"""GPU edge cases at the engine's limits.

- The largest draft window (31 tokens, 32 verify rows) against the oracle.
- 64-row verifies (several launches of either decode kernel): every row
  equal to the greedy step at its position, bit for bit.
- The KV-capacity boundary of a generation.
- Grouped-query attention with 8 query heads per KV head (the 70B grouping)
  on a small bf16 model: logits against the oracle, speculative == greedy,
  batched == single-sequence runs.
"""
import numpy as np
import pytest

import lss_synth
import oracle
from lss_synth.shapes import ModelShape

pytestmark = pytest.mark.gpu

GQA8 = ModelShape("gqa8_bf16", 2, 512, 8, 1, 64, 1024, 2048, 1e4, "bf16", weight_seed=21, prompt_seed=121)


@pytest.fixture(scope="module")
def tiny():
    from layer_skip_self_amd import Engine
    sh = lss_synth.SHAPES["tiny"]
    w_cpu = lss_synth.make_weights(sh, device="cpu")
    w_gpu = [(n, t.to("cuda")) for n, t in w_cpu]
    model = oracle.OracleModel(sh, lss_synth.weights_to_numpy(w_cpu))
    yield dict(sh=sh, w=w_gpu, model=model, prompt=lss_synth.make_prompt(sh, 32))


def test_largest_window_matches_oracle(tiny):
    from layer_skip_self_amd import Engine
    G = 80
    eng = Engine(tiny["sh"], tiny["w"], max_seq=32 + G + 33, max_rows=32)
    try:
        ar, _ = eng.generate(tiny["prompt"], G, {"mode": "ar"})
        toks, st = eng.generate(tiny["prompt"], G, {"mode": "static", "k_max": 31, "skip": (1, 2)})
    finally:
        eng.close()
    ref, recs = oracle.speculative_generate(tiny["model"], tiny["prompt"], G, oracle.Policy(K=31, skip=(1, 2)))
    print(f"K 31: {st}")
    assert toks == ar == ref
    assert st["rounds"] == len(recs)
    assert st["accepted"] == sum(r["n"] for r in recs)
    assert max(r["k"] for r in recs) == 31


@pytest.mark.parametrize("kernel", ["vector", "mfma"])
def test_64_row_verify_rows_equal_greedy_steps(kernel):
    """31 drafts on a 64-row engine: the vector GEMV takes 8 rows per launch
    at these depths, the MFMA GEMM 16; every row equals the greedy step."""
    from layer_skip_self_amd import Engine
    sh = lss_synth.SHAPES["small_bf16"]
    w = lss_synth.make_weights(sh, device="cuda")
    prompt = lss_synth.make_prompt(sh, 40)
    eng = Engine(sh, w, max_seq=160, max_rows=64)
    try:
        eng.set_decode_kernel(kernel)
        toks = [eng.prefill(prompt)]
        zs = []
        for _ in range(31):
            eng.verify(None, 0)
            zs.append(eng.read_logits(1)[0].copy())
            toks.append(eng.accept()[1])
        eng.verify(None, 0)
        zs.append(eng.read_logits(1)[0].copy())
        eng.accept()
        eng.prefill(prompt)
        eng.verify(drafts=toks[1:32])
        zv = eng.read_logits(32)
        n, _, _ = eng.accept()
        assert n == 31
        for i in range(32):
            assert np.array_equal(zv[i], zs[i]), f"row {i}"
    finally:
        eng.close()


def test_kv_capacity_boundary(tiny):
    from layer_skip_self_amd import Engine
    from layer_skip_self_amd.engine import LssError
    G, R = 16, 16
    need = 32 + G + min(31, R - 1) + 1
    pol = {"mode": "static", "k_max": 6, "skip": (1,)}
    eng = Engine(tiny["sh"], tiny["w"], max_seq=need, max_rows=R)
    try:
        ar, _ = eng.generate(tiny["prompt"], G, {"mode": "ar"})
        toks, _ = eng.generate(tiny["prompt"], G, pol)
        assert toks == ar
    finally:
        eng.close()
    eng = Engine(tiny["sh"], tiny["w"], max_seq=need - 1, max_rows=R)
    try:
        with pytest.raises(LssError):
            eng.generate(tiny["prompt"], G, pol)
    finally:
        eng.close()


@pytest.fixture(scope="module")
def gqa8():
    from layer_skip_self_amd import Engine
    w_cpu = lss_synth.make_weights(GQA8, device="cpu")
    w_gpu = [(n, t.to("cuda")) for n, t in w_cpu]
    model = oracle.OracleModel(GQA8, lss_synth.weights_to_numpy(w_cpu))
    eng = Engine(GQA8, w_gpu, max_seq=200, max_rows=32, max_seqs=3)
    one = Engine(GQA8, w_gpu, max_seq=200, max_rows=32)
    yield dict(model=model, eng=eng, one=one)
    eng.close()
    one.close()


def test_gqa8_logits_match_oracle(gqa8):
    """Prefill and a 9-row teacher-forced verify (the oracle's greedy tokens)
    against the oracle at the bf16 bound."""
    import copy
    prompt = lss_synth.make_prompt(GQA8, 48)
    one, model = gqa8["one"], gqa8["model"]
    t0 = one.prefill(prompt)
    z0 = one.read_logits(1)[0]
    st, zr, _ = oracle.prefill(model, prompt, 200)
    assert np.max(np.abs(z0 - zr)) <= 2e-2
    assert t0 == st.t0
    so = copy.deepcopy(st)
    toks, ref = [st.t0], []
    for _ in range(9):
        z, _ = oracle.forward_row(model, so, toks[-1], so.p, "full")
        so.p += 1
        ref.append(z)
        toks.append(int(np.argmax(z)))
    one.verify(drafts=toks[1:9])
    zv = one.read_logits(9)
    one.accept()
    err = float(np.max(np.abs(zv - np.stack(ref))))
    print(f"GQA 8 verify rows: max error {err:.3g}")
    assert err <= 2e-2


@pytest.mark.parametrize("kernel", ["vector", "mfma_verify"])
def test_gqa8_batch_and_speculative_equal_greedy(gqa8, kernel):
    rng = np.random.default_rng(3)
    prompts = [rng.integers(0, GQA8.vocab, n).astype(np.int32) for n in (48, 21, 70)]
    pol = {"mode": "dp", "k_max": 5, "n_skip": 1, "interval": 3, "decode_kernel": kernel}
    try:
        toks, stats = gqa8["eng"].generate_batch(prompts, 40, pol)
        ar, _ = gqa8["eng"].generate_batch(prompts, 40, {"mode": "ar", "decode_kernel": kernel})
        for i, p in enumerate(prompts):
            single, st = gqa8["one"].generate(p, 40, pol)
            assert toks[i] == single == ar[i], i
            assert stats[i] == st, i
    finally:
        gqa8["eng"].set_decode_kernel("vector")
        gqa8["one"].set_decode_kernel("vector")
