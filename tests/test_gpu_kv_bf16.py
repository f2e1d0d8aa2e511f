"""GPU parity of the bf16 KV cache (``kv_dtype="bf16"``) against the oracle
with the same cache (``OracleModel(..., kv_dtype="bf16")``: keys and values
rounded to bfloat16 where the cache holds them and where a row uses its own).

Two models: the 4-layer float32 model (head dim 64, MHA) and the small bf16
model (3 layers, 5 query heads on 1 kv head, ragged projection depths).
Checked against the oracle: prefill logits, greedy decode along the GPU's
own tokens (the parity protocol's token rule), and teacher-forced verify
rows.  Checked on the GPU alone: every verify row equals the greedy step at
its position bit for bit, and speculative output equals greedy output for
chain, DP and tree drafts.  Batched sequences (the batched attention kernels
on a bf16 cache) equal both the oracle's and the GPU's single-sequence runs."""
import numpy as np
import pytest

import lss_synth
import oracle

pytestmark = pytest.mark.gpu

G = 40
# tolerance per model: float32 weights (4-layer model) keep the oracle's
# 1e-4; the bf16 model's activations carry ~16 bits on the GPU (2e-3, as in
# its float32-cache tests).  A key or value whose float32 value lies within
# rounding distance of a bfloat16 midpoint may round the other way on one
# side; such flips move a logit by far less than these bounds.
CASES = {"tiny": 1e-4, "small_bf16": 2e-3}


@pytest.fixture(scope="module", params=sorted(CASES))
def case(request):
    from layer_skip_self_amd import Engine
    name = request.param
    shape = lss_synth.SHAPES[name]
    w_cpu = lss_synth.make_weights(shape, device="cpu")
    w_gpu = [(n, t.to("cuda")) for n, t in w_cpu]
    model = oracle.OracleModel(shape, lss_synth.weights_to_numpy(w_cpu), kv_dtype="bf16")
    prompt = lss_synth.make_prompt(shape, 36)
    eng = Engine(shape, w_gpu, max_seq=160, max_rows=16, kv_dtype="bf16")
    st, z, _ = oracle.prefill(model, prompt, 160)
    ref, ref_z = [st.t0], [z]
    st_ref = st
    import copy
    st = copy.deepcopy(st_ref)
    while len(ref) < G:
        zz, _ = oracle.forward_row(model, st, st.t0, st.p, "full")
        st.p += 1
        st.t0 = int(np.argmax(zz))
        ref.append(st.t0)
        ref_z.append(zz)
    yield dict(name=name, tol=CASES[name], model=model, prompt=prompt, eng=eng, ref=ref, ref_z=ref_z,
               st0=st_ref, z0=z)
    eng.close()


def test_prefill_and_greedy_ids_vs_oracle(case):
    from conftest import greedy_ids_vs_oracle
    eng = case["eng"]
    n, total, worst = greedy_ids_vs_oracle(eng, case["model"], case["prompt"], case["st0"], case["z0"], G - 1,
                                           case["tol"])
    print(f"{case['name']}: {n} of {total} ids compared, logits max-abs {worst:.3e}")
    assert n >= total - 4


@pytest.mark.parametrize("rows", [2, 5, 9])
def test_teacher_forced_verify_rows_vs_oracle(case, rows):
    eng, ref, ref_z = case["eng"], case["ref"], case["ref_z"]
    eng.prefill(case["prompt"])
    eng.verify(drafts=ref[1:rows])
    z = eng.read_logits(rows)
    eng.accept()
    err = float(np.max(np.abs(z - np.stack(ref_z[1:rows + 1]))))
    print(f"{case['name']} {rows} rows: max-abs {err:.3e}")
    assert err <= case["tol"]


def test_verify_rows_equal_greedy_steps_bitwise(case):
    eng, prompt = case["eng"], case["prompt"]
    eng.prefill(prompt)
    ar_z, toks = [], []
    for _ in range(9):
        eng.verify(None, 0)
        ar_z.append(eng.read_logits(1)[0].copy())
        _, b, _ = eng.accept()
        toks.append(b)
    eng.prefill(prompt)
    eng.verify(drafts=toks[:8])
    z = eng.read_logits(9)
    for i in range(9):
        assert np.array_equal(z[i].view(np.uint32), ar_z[i].view(np.uint32)), i
    n, _, _ = eng.accept()
    assert n == 8


POLICIES = {
    "static_K6": {"mode": "static", "k_max": 6, "skip": (1,)},
    "dp_S1_I3": {"mode": "dp", "k_max": 5, "n_skip": 1, "interval": 3},
    "tree_B3_D3": {"mode": "dp", "k_max": 1, "n_skip": 1, "interval": 4, "tree_width": 3, "tree_depth": 3},
}


@pytest.mark.parametrize("name", sorted(POLICIES))
def test_speculative_equals_greedy(case, name):
    eng, prompt = case["eng"], case["prompt"]
    ar, _ = eng.generate(prompt, G, {"mode": "ar"})
    toks, st = eng.generate(prompt, G, POLICIES[name])
    assert toks == ar
    assert 0 <= st["accepted"] <= st["drafted"]


def test_batched_sequences_with_bf16_cache(case):
    """Three sequences decoded together with a bf16 cache (the batched
    attention kernels on bf16 keys and values) equal the oracle's
    single-sequence runs with the same cache, and the GPU's own single runs."""
    from layer_skip_self_amd import Engine
    shape = lss_synth.SHAPES[case["name"]]
    w_gpu = [(n, t.to("cuda")) for n, t in lss_synth.make_weights(shape, device="cpu")]
    rng = np.random.default_rng(17)
    prompts = [rng.integers(0, shape.vocab, m).astype(np.int32) for m in (30, 17, 41)]
    eng = Engine(shape, w_gpu, max_seq=120, max_rows=16, kv_dtype="bf16", max_seqs=3)
    try:
        for gp, op in (({"mode": "ar"}, oracle.Policy(K=0)),
                       ({"mode": "static", "k_max": 4, "skip": (1,)}, oracle.Policy(K=4, skip=(1,)))):
            toks, _ = eng.generate_batch(prompts, 24, gp)
            ref = oracle.batch_generate(case["model"], prompts, 24, op)
            for i, p in enumerate(prompts):
                single, _ = case["eng"].generate(p, 24, gp)
                assert toks[i] == single, (gp["mode"], i)
                assert toks[i] == ref[i][0], (gp["mode"], i)
    finally:
        eng.close()
