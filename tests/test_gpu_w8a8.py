"""GPU parity of the W8A8 draft (int8 weight copy + int8 activations).

Bit-exact against the oracle: the weight quantizer (codes and scales) and
the int8 GEMV (exact integer accumulation, then two float32 products), over
shapes with several tiles, a ragged K (not a multiple of the 1 KB chunk) and
the 8B shapes.  Through the engine on the 4-layer model: a W8A8 draft step's
logits against the oracle's, and speculative output equal to greedy output
bit for bit for W8A8 drafts (static, exit threshold, DP, cascade levels).
"""
import numpy as np
import pytest

import lss_synth
import oracle
from oracle.model import quantize_weight_rows, w8a8_accumulate

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,k", [(48, 688), (512, 4096), (64, 14336)])
def test_weight_quantizer_bitexact(dtype, rows, k):
    import torch
    from layer_skip_self_amd.engine import w8_quantize
    g = torch.Generator(device="cpu").manual_seed(rows * 7 + k)
    w = torch.randn(rows, k, generator=g) * 0.02
    w[3] = 0.0                                   # amax = 0 row
    w[5, 7] = 0.75                               # one dominant element
    w = w.to(torch.bfloat16 if dtype == "bf16" else torch.float32)
    q, s = w8_quantize(w.to("cuda"))
    torch.cuda.synchronize()
    Q, S = quantize_weight_rows(w.float().numpy())
    assert np.array_equal(q.cpu().numpy(), Q)
    assert np.array_equal(s.cpu().numpy(), S)


@pytest.mark.parametrize("n,k", [(64, 688), (6144, 4096), (4096, 14336), (256, 16), (128, 28672)])
def test_w8a8_gemv_bitexact(n, k):
    import torch
    from layer_skip_self_amd.engine import w8a8_gemv
    rng = np.random.default_rng(n + k)
    Q = rng.integers(-127, 128, (n, k)).astype(np.int8)
    q = rng.integers(-127, 128, k).astype(np.int8)
    Q[0] = 127
    q[:] = np.where(np.arange(k) % 2 == 0, q, 127)
    Q[1] = -127                                  # large accumulators of both signs
    ws = (rng.random(n).astype(np.float32) * np.float32(1e-3)).astype(np.float32)
    xs = np.array([0.0173], np.float32)
    y = w8a8_gemv(torch.from_numpy(Q).cuda(), torch.from_numpy(ws).cuda(), torch.from_numpy(q).cuda(),
                  torch.from_numpy(xs).cuda())
    torch.cuda.synchronize()
    acc = w8a8_accumulate(Q, q)
    ref = (acc.astype(np.float32) * (ws * xs[0]).astype(np.float32)).astype(np.float32)
    got = y.cpu().numpy()
    assert np.array_equal(got, ref), np.max(np.abs(got - ref))


@pytest.mark.parametrize("n,k", [(64, 688), (6144, 4096), (4096, 14336), (256, 16), (128, 8192), (64, 28672)])
def test_w8a8_gemv_with_in_kernel_quantization_bitexact(n, k):
    """Every workgroup quantizes the float32 row itself (the draft's form):
    equal bit for bit to the oracle's w8a8_project (codes decided in float32
    by the per-token rule, exact accumulation, two float32 products)."""
    import torch
    from layer_skip_self_amd.engine import w8a8_gemv_f32
    from oracle.model import w8a8_project
    rng = np.random.default_rng(3 * n + k)
    W = (rng.normal(0, 0.02, (n, k))).astype(np.float32)
    Q, S = quantize_weight_rows(W)
    x = rng.normal(0, 1.0, k).astype(np.float32)
    x[k // 3] = 4.0                               # a dominant element sets amax
    y = w8a8_gemv_f32(torch.from_numpy(Q).cuda(), torch.from_numpy(S).cuda(), torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    ref = w8a8_project(Q, S, x)
    got = y.cpu().numpy()
    assert np.array_equal(got, ref), np.max(np.abs(got - ref))


@pytest.fixture(scope="module")
def tiny():
    from layer_skip_self_amd import Engine
    shape = lss_synth.SHAPES["tiny"]
    w_cpu = lss_synth.make_weights(shape, device="cpu")
    w_gpu = [(n, t.to("cuda")) for n, t in w_cpu]
    model = oracle.OracleModel(shape, lss_synth.weights_to_numpy(w_cpu))
    prompt = lss_synth.make_prompt(shape, 32)
    eng = Engine(shape, w_gpu, max_seq=256, max_rows=16)
    eng.attach_w8()
    yield dict(shape=shape, model=model, prompt=prompt, eng=eng)
    eng.close()


def test_w8a8_draft_logits_vs_oracle(tiny):
    eng, model, prompt = tiny["eng"], tiny["model"], tiny["prompt"]
    for mask in ([0, 0, 0, 0], [0, 1, 1, 0]):
        eng.prefill(prompt)
        d = eng.draft(mask, 2, 3)
        st, _, _ = oracle.prefill(model, prompt, 256)
        od, _ = oracle.draft(model, st, mask, 2, 3)
        assert d == od
        # last step's logits: re-run the oracle's third step's row
        zg = eng.read_logits(1)[0]
        st2, _, _ = oracle.prefill(model, prompt, 256)
        oracle.draft(model, st2, mask, 2, 2)
        zo, _ = oracle.forward_row(model, st2, st2.window[-1], st2.p + 2, "draft", mask, 2)
        err = float(np.max(np.abs(zg - zo)))
        print(f"mask {mask}: W8A8 draft logits max-abs {err:.3e}")
        assert err <= 1e-3
        eng.verify(k=len(d))
        eng.accept()


def test_engine_refuses_w8a8_without_copy():
    from layer_skip_self_amd import Engine
    from layer_skip_self_amd.engine import LssError
    shape = lss_synth.SHAPES["tiny"]
    w = lss_synth.make_weights(shape, device="cuda")
    eng = Engine(shape, w, max_seq=128, max_rows=8)
    eng.prefill(lss_synth.make_prompt(shape, 16))
    with pytest.raises(LssError):
        eng.draft([0, 0, 0, 0], 2, 1)
    eng.close()


G = 64
POLICIES = {
    "static_12_K4": {"mode": "static", "k_max": 4, "skip": (1, 2), "quant": 2},
    "empty_mask_K6": {"mode": "static", "k_max": 6, "skip": (), "quant": 2},
    "tau_skip2_K5": {"mode": "static", "k_max": 5, "skip": (2,), "exit_tau": 0.3, "quant": 2},
    "dp_S2_I4": {"mode": "dp", "k_max": 4, "n_skip": 2, "interval": 4, "quant": 2},
    "cascade": {"mode": "cascade", "k_max": 8, "interval": 5, "levels": [(3, 1, 2), (1, 0, 2), (0, 0, 1)],
                "beta": (0.1, 0.0, 0.05)},
}


@pytest.mark.parametrize("name", sorted(POLICIES))
def test_w8a8_speculative_equals_greedy(tiny, name):
    eng = tiny["eng"]
    ar, _ = eng.generate(tiny["prompt"], G, {"mode": "ar"})
    toks, st = eng.generate(tiny["prompt"], G, POLICIES[name])
    print(f"{name}: accepted {st['accepted']} of {st['drafted']}")
    assert toks == ar
    assert st["accepted"] > 0
