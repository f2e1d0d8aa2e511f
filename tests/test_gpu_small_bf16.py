"""GPU parity of the bf16 decode kernels on a small bf16 model (3 layers,
d 320, 5 query heads / 1 kv head of 64, FFN 864, vocab 1008) whose
projection depths (320, 864) end in ragged 128-element pieces and leave
some waves of a decode launch without work.  Every decode-kernel setting
(the vector-ALU GEMV, the MFMA GEMM, MFMA for full-model rows only) is
checked:

  * against the float64 oracle (on the bf16-rounded weights): prefill,
    decode steps along the GPU's own tokens, and verify passes of 2 .. 16
    rows teacher-forced on the oracle's tokens;
  * the GPU's own losslessness: every verify row equals the greedy step at
    its position bit for bit, speculative output equals greedy output for
    several policies (windows up to 15 drafts, int8 drafts), and the grid
    policy of the decode launch changes no bit."""
import numpy as np
import pytest

import lss_synth
import oracle

pytestmark = pytest.mark.gpu

SHAPE = lss_synth.SHAPES["small_bf16"]
G = 48
TOL = 2e-3      # bf16 weights are exact on both sides; activations carry ~16 bits on the GPU


@pytest.fixture(scope="module")
def small():
    from layer_skip_self_amd import Engine
    w_cpu = lss_synth.make_weights(SHAPE, device="cpu")
    w_gpu = [(n, t.to("cuda")) for n, t in w_cpu]
    model = oracle.OracleModel(SHAPE, lss_synth.weights_to_numpy(w_cpu))
    prompt = lss_synth.make_prompt(SHAPE, 40)
    eng = Engine(SHAPE, w_gpu, max_seq=160, max_rows=16)
    st, z, _ = oracle.prefill(model, prompt, 160)
    ref, ref_z = [st.t0], [z]
    while len(ref) < G:
        zz, _ = oracle.forward_row(model, st, st.t0, st.p, "full")
        st.p += 1
        st.t0 = int(np.argmax(zz))
        ref.append(st.t0)
        ref_z.append(zz)
    yield dict(model=model, prompt=prompt, eng=eng, ref=ref, ref_z=ref_z)
    eng.close()


@pytest.fixture(params=["mfma", "vector", "mfma_verify"])
def kernel(small, request):
    small["eng"].set_decode_kernel(request.param)
    yield request.param
    small["eng"].set_decode_kernel("vector")


def test_prefill_and_decode_steps_vs_oracle(small, kernel):
    from conftest import greedy_ids_vs_oracle
    st0, z0, _ = oracle.prefill(small["model"], small["prompt"], 160)
    n, total, worst = greedy_ids_vs_oracle(small["eng"], small["model"], small["prompt"], st0, z0, G - 1, TOL)
    print(f"{kernel}: {n} of {total} ids compared, logits max-abs {worst:.3e}")
    assert n >= total - 4


@pytest.mark.parametrize("rows", [2, 3, 5, 9, 16])
def test_teacher_forced_verify_rows_vs_oracle(small, kernel, rows):
    eng, ref, ref_z = small["eng"], small["ref"], small["ref_z"]
    eng.prefill(small["prompt"])
    eng.verify(drafts=ref[1:rows])
    z = eng.read_logits(rows)
    n, _, _ = eng.accept()
    err = float(np.max(np.abs(z - np.stack(ref_z[1:rows + 1]))))
    print(f"{kernel} {rows} rows: max-abs {err:.3e}, {n} accepted")
    assert err <= TOL


def test_verify_rows_equal_greedy_steps_bitwise(small, kernel):
    """Every row of verifies of 16, 9, 5, 2 rows equals the one-row greedy
    step at its position (logits and residual states, bit for bit)."""
    eng, prompt = small["eng"], small["prompt"]
    eng.prefill(prompt)
    ar_z, ar_h, toks = [], [], []
    for _ in range(16):
        eng.verify(None, 0)
        ar_z.append(eng.read_logits(1)[0].copy())
        ar_h.append(eng.read_states(0))
        _, b, _ = eng.accept()
        toks.append(b)
    for rows in (16, 9, 5, 2):
        eng.prefill(prompt)
        eng.verify(drafts=toks[:rows - 1])
        z = eng.read_logits(rows)
        for i in range(rows):
            assert np.array_equal(z[i].view(np.uint32), ar_z[i].view(np.uint32)), (rows, i)
            assert np.array_equal(eng.read_states(i).view(np.uint32), ar_h[i].view(np.uint32)), (rows, i)
        n, _, _ = eng.accept()
        assert n == rows - 1


POLICIES = {
    "static_K15": {"mode": "static", "k_max": 15, "skip": (1,)},
    "empty_mask_K8": {"mode": "static", "k_max": 8, "skip": ()},
    "quant_K6": {"mode": "static", "k_max": 6, "skip": (2,), "quant": 1},
    "dp_S1_I3": {"mode": "dp", "k_max": 5, "n_skip": 1, "interval": 3},
    "tree_B4": {"mode": "dp", "k_max": 1, "n_skip": 1, "interval": 4, "tree_width": 4},
    "tree_B3_D4": {"mode": "dp", "k_max": 1, "n_skip": 1, "interval": 4, "tree_width": 3, "tree_depth": 4},
    "tree_empty_mask_B2_D5": {"mode": "static", "k_max": 1, "skip": (), "tree_width": 2, "tree_depth": 5},
}


@pytest.mark.parametrize("name", sorted(POLICIES))
def test_speculative_equals_greedy(small, kernel, name):
    eng, prompt = small["eng"], small["prompt"]
    ar, _ = eng.generate(prompt, G, {"mode": "ar"})
    toks, st = eng.generate(prompt, G, POLICIES[name])
    assert toks == ar
    if name == "empty_mask_K8" and kernel != "mfma_verify":
        assert st["accepted"] == st["drafted"]     # the draft is the full model bit for bit
    if name == "tree_empty_mask_B2_D5" and kernel != "mfma_verify":
        # the full-model draft's first branch is the greedy continuation: every
        # round accepts its whole depth (drafted counts both branches' nodes)
        assert 2 * st["accepted"] == st["drafted"]


def test_grid_policies_bitwise_equal(small, kernel):
    eng, prompt, ref = small["eng"], small["prompt"], small["ref"]
    out = None
    try:
        for g in (1, 0, 3, 8):
            eng.set_gemv_grid(g)
            eng.prefill(prompt)
            eng.verify(drafts=ref[1:12])
            z = eng.read_logits(12)
            hs = eng.read_states(11)
            eng.accept()
            if out is None:
                out = (z, hs)
            else:
                assert np.array_equal(z.view(np.uint32), out[0].view(np.uint32)), g
                assert np.array_equal(hs.view(np.uint32), out[1].view(np.uint32)), g
    finally:
        eng.set_gemv_grid(1)


def test_draft_steps_vs_oracle(small, kernel):
    """Draft steps with a skip mask, full precision and int8 activations."""
    eng, model, prompt = small["eng"], small["model"], small["prompt"]
    for quant, tol in [(0, TOL), (1, 3e-2)]:
        mask = [0, 1, 0]
        eng.prefill(prompt)
        st, _, _ = oracle.prefill(model, prompt, 160)
        for s in range(3):
            g = eng.draft(mask, quant, 1)
            zg = eng.read_logits(1)[0]
            tok_o = st.t0 if not st.window else st.window[-1]
            zo, _ = oracle.forward_row(model, st, tok_o, st.p + len(st.window), "draft", mask, quant)
            st.window.append(int(np.argmax(zo)))
            err = float(np.max(np.abs(zg - zo)))
            print(f"{kernel} quant={quant} step {s}: max-abs {err:.3e}")
            assert err <= tol
            if oracle.argmax_first(zo) != g[0]:
                break
        eng.verify(None, s + 1)
        eng.accept()
