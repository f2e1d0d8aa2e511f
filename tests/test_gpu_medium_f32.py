"""GPU parity of the float32-weight decode kernels at real projection depths:
a 2-layer float32 model (d 1024, 8 query / 2 kv heads of 128, FFN 5632,
vocab 4096).  Its FFN depth is 22 chunks of 1 KB of float32 weights, so the
down projection's GEMV gives each wave 3 or 2 chunks (four chunk registers,
at most 4 rows per launch: a 9-row verify runs as 4 + 4 + 1 rows), while the
depth-1024 projections keep one chunk per wave (8-row launches); attention
runs at head dim 128 with GQA 4 on a float32 cache.

Against the float64 oracle: prefill, greedy decode along the GPU's own
tokens (the parity protocol's token rule) and teacher-forced verify rows.
On the GPU alone: verify rows equal greedy steps bit for bit (also across
the row-group launches), and speculative output equals greedy output.  A
one-layer wide float32 model (d 3072, FFN 14336) covers the two- and
eight-chunk GEMV variants (2-row launches) the same way."""
import numpy as np
import pytest

import lss_synth
import oracle

pytestmark = pytest.mark.gpu

SHAPE = lss_synth.SHAPES["medium_f32"]
G = 32
TOL = 1e-4      # float32 weights on both sides; the GPU accumulates in float32


@pytest.fixture(scope="module")
def medium():
    import copy
    from layer_skip_self_amd import Engine
    w_cpu = lss_synth.make_weights(SHAPE, device="cpu")
    w_gpu = [(n, t.to("cuda")) for n, t in w_cpu]
    model = oracle.OracleModel(SHAPE, lss_synth.weights_to_numpy(w_cpu))
    prompt = lss_synth.make_prompt(SHAPE, 48)
    eng = Engine(SHAPE, w_gpu, max_seq=128, max_rows=16)
    st0, z0, _ = oracle.prefill(model, prompt, 128)
    st = copy.deepcopy(st0)
    ref, ref_z = [st.t0], [z0]
    while len(ref) < G:
        zz, _ = oracle.forward_row(model, st, st.t0, st.p, "full")
        st.p += 1
        st.t0 = int(np.argmax(zz))
        ref.append(st.t0)
        ref_z.append(zz)
    yield dict(model=model, prompt=prompt, eng=eng, ref=ref, ref_z=ref_z, st0=st0, z0=z0)
    eng.close()


def test_prefill_and_greedy_ids_vs_oracle(medium):
    from conftest import greedy_ids_vs_oracle
    n, total, worst = greedy_ids_vs_oracle(medium["eng"], medium["model"], medium["prompt"], medium["st0"],
                                           medium["z0"], G - 1, TOL)
    print(f"{n} of {total} ids compared, logits max-abs {worst:.3e}")
    assert n >= total - 4


@pytest.mark.parametrize("rows", [2, 4, 5, 9])
def test_teacher_forced_verify_rows_vs_oracle(medium, rows):
    eng, ref, ref_z = medium["eng"], medium["ref"], medium["ref_z"]
    eng.prefill(medium["prompt"])
    eng.verify(drafts=ref[1:rows])
    z = eng.read_logits(rows)
    eng.accept()
    err = float(np.max(np.abs(z - np.stack(ref_z[1:rows + 1]))))
    print(f"{rows} rows: max-abs {err:.3e}")
    assert err <= TOL


def test_verify_rows_equal_greedy_steps_bitwise(medium):
    eng, prompt = medium["eng"], medium["prompt"]
    eng.prefill(prompt)
    ar_z, ar_h, toks = [], [], []
    for _ in range(9):
        eng.verify(None, 0)
        ar_z.append(eng.read_logits(1)[0].copy())
        ar_h.append(eng.read_states(0))
        _, b, _ = eng.accept()
        toks.append(b)
    for rows in (9, 5, 2):
        eng.prefill(prompt)
        eng.verify(drafts=toks[:rows - 1])
        z = eng.read_logits(rows)
        for i in range(rows):
            assert np.array_equal(z[i].view(np.uint32), ar_z[i].view(np.uint32)), (rows, i)
            assert np.array_equal(eng.read_states(i).view(np.uint32), ar_h[i].view(np.uint32)), (rows, i)
        n, _, _ = eng.accept()
        assert n == rows - 1


POLICIES = {
    "static_K8": {"mode": "static", "k_max": 8, "skip": (1,)},
    "empty_mask_K6": {"mode": "static", "k_max": 6, "skip": ()},
    "quant_K4": {"mode": "static", "k_max": 4, "skip": (0,), "quant": 1},
    "dp_S1_I3": {"mode": "dp", "k_max": 5, "n_skip": 1, "interval": 3},
    "tree_B3_D3": {"mode": "dp", "k_max": 1, "n_skip": 1, "interval": 4, "tree_width": 3, "tree_depth": 3},
}


@pytest.mark.parametrize("name", sorted(POLICIES))
def test_speculative_equals_greedy(medium, name):
    eng, prompt = medium["eng"], medium["prompt"]
    ar, _ = eng.generate(prompt, G, {"mode": "ar"})
    toks, st = eng.generate(prompt, G, POLICIES[name])
    assert toks == ar
    if name == "empty_mask_K6":
        assert st["accepted"] == st["drafted"]     # the draft is the full model bit for bit


# ---------------------------------------------------------------- wide float32 model (one layer)
WIDE = lss_synth.SHAPES["wide_f32"]


@pytest.fixture(scope="module")
def wide():
    import copy
    from layer_skip_self_amd import Engine
    w_cpu = lss_synth.make_weights(WIDE, device="cpu")
    w_gpu = [(n, t.to("cuda")) for n, t in w_cpu]
    model = oracle.OracleModel(WIDE, lss_synth.weights_to_numpy(w_cpu))
    prompt = lss_synth.make_prompt(WIDE, 40)
    eng = Engine(WIDE, w_gpu, max_seq=96, max_rows=16)
    st0, z0, _ = oracle.prefill(model, prompt, 96)
    st = copy.deepcopy(st0)
    ref, ref_z = [st.t0], [z0]
    while len(ref) < 12:
        zz, _ = oracle.forward_row(model, st, st.t0, st.p, "full")
        st.p += 1
        st.t0 = int(np.argmax(zz))
        ref.append(st.t0)
        ref_z.append(zz)
    yield dict(model=model, prompt=prompt, eng=eng, ref=ref, ref_z=ref_z, st0=st0, z0=z0)
    eng.close()


def test_wide_greedy_and_verify_rows_vs_oracle(wide):
    """Two and eight chunk registers per wave (depths 3072 and 14336): greedy
    ids and logits along the GPU's tokens, and a 9-row verify (its down
    projection in five 2-row launches) teacher-forced on the oracle's."""
    from conftest import greedy_ids_vs_oracle
    eng = wide["eng"]
    n, total, worst = greedy_ids_vs_oracle(eng, wide["model"], wide["prompt"], wide["st0"], wide["z0"], 11, TOL)
    print(f"wide: {n} of {total} ids compared, logits max-abs {worst:.3e}")
    assert n >= total - 2
    eng.prefill(wide["prompt"])
    eng.verify(drafts=wide["ref"][1:9])
    z = eng.read_logits(9)
    eng.accept()
    err = float(np.max(np.abs(z - np.stack(wide["ref_z"][1:10]))))
    print(f"wide 9 rows: max-abs {err:.3e}")
    assert err <= TOL


def test_wide_verify_rows_equal_greedy_steps_bitwise(wide):
    eng, prompt = wide["eng"], wide["prompt"]
    eng.prefill(prompt)
    ar_z, toks = [], []
    for _ in range(9):
        eng.verify(None, 0)
        ar_z.append(eng.read_logits(1)[0].copy())
        _, b, _ = eng.accept()
        toks.append(b)
    for rows in (9, 3):
        eng.prefill(prompt)
        eng.verify(drafts=toks[:rows - 1])
        z = eng.read_logits(rows)
        for i in range(rows):
            assert np.array_equal(z[i].view(np.uint32), ar_z[i].view(np.uint32)), (rows, i)
        n, _, _ = eng.accept()
        assert n == rows - 1
    ar, _ = eng.generate(prompt, 24, {"mode": "ar"})
    toks, st = eng.generate(prompt, 24, {"mode": "static", "k_max": 6, "skip": ()})
    assert toks == ar and st["accepted"] == st["drafted"]
    toks, _ = eng.generate(prompt, 24, {"mode": "static", "k_max": 4, "skip": (), "quant": 1})
    assert toks == ar
