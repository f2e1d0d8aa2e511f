"""GPU parity at the Llama-3-70B shape on one GPU (80 layers, d 8192, 64 q /
8 kv heads, FFN 28672, vocab 128256, bf16, ~141 GB of weights in HBM).

The float32 oracle cannot hold this model on the host, so parity is taken in
per-layer slices: a 64-token prompt (one prefill block) leaves every row's
residual state after every layer in the engine's stash; for sampled layers
the oracle runs that one layer (``oracle.layer_block``) on the GPU's input
rows and is compared with the GPU's output rows; the last row's logits are
compared after the oracle's final norm and LM head.  Tolerance 2e-2 (bf16).
Property at the full shape: speculative decoding with the 70B policy (the
CLaSp DP skipping 44 of 80 layers, K = 8) equals greedy decoding bit for
bit."""
import numpy as np
import pytest

import lss_synth
import oracle

pytestmark = pytest.mark.gpu

SHAPE = lss_synth.SHAPES["llama3_70b"]
P = 64
MAX_SEQ = 512 + 256 + 33
TOL = 2e-2
SLICES = (0, 41, 79)


@pytest.fixture(scope="module")
def gpu70b():
    import time
    import torch
    from layer_skip_self_amd import Engine
    t = time.time()
    w = lss_synth.make_weights(SHAPE, device="cuda")
    torch.cuda.synchronize()
    print(f"\n70B weights generated in {time.time() - t:.1f} s", flush=True)
    eng = Engine(SHAPE, w, max_seq=MAX_SEQ, max_rows=64)
    prompt = lss_synth.make_prompt(SHAPE, P)
    yield dict(w=w, eng=eng, prompt=prompt)
    eng.close()


@pytest.fixture(scope="module")
def slice_model(gpu70b):
    """Oracle over host copies of the sampled layers and the head only."""
    keep = {"final_norm", "lm_head"} | {f"layers.{l}.{n}" for l in SLICES
                                        for n in ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm",
                                                  "w_gate", "w_up", "w_down")}
    w_host = [(n, t.to("cpu")) for n, t in gpu70b["w"] if n in keep]
    return oracle.OracleModel(SHAPE, lss_synth.LazyF32(w_host), dtype=np.float32, cache_layers=False)


def test_layer_slices_and_logits_vs_oracle_70b(gpu70b, slice_model):
    eng = gpu70b["eng"]
    eng.prefill(gpu70b["prompt"])
    z = eng.read_logits(1)[0]
    states = np.stack([eng.read_states(r) for r in range(P)])      # [P][L+1][d]
    for l in SLICES:
        ref = oracle.layer_block(slice_model, l, states[:, l, :].astype(np.float32))
        err = float(np.max(np.abs(states[:, l + 1, :] - ref)))
        print(f"layer {l}: max-abs {err:.3e} (max |h| {np.max(np.abs(ref)):.3f})", flush=True)
        assert err <= TOL
    zo = slice_model.head(states[P - 1, SHAPE.n_layers, :].astype(np.float32))
    err = float(np.max(np.abs(z - zo)))
    print(f"last-row logits max-abs {err:.3e}", flush=True)
    assert err <= TOL


def test_speculative_equals_greedy_bitwise_70b(gpu70b):
    eng, prompt = gpu70b["eng"], gpu70b["prompt"]
    G = 24
    ar, _ = eng.generate(prompt, G, {"mode": "ar"})
    toks, st = eng.generate(prompt, G, {"mode": "dp", "k_max": 8, "n_skip": 44, "interval": 8})
    assert toks == ar
    assert st["dp_runs"] >= 1
    # with the MFMA GEMM for the full-model rows (one launch per 9-row verify)
    eng.set_decode_kernel("mfma_verify")
    try:
        ar2, _ = eng.generate(prompt, G, {"mode": "ar"})
        toks2, _ = eng.generate(prompt, G, {"mode": "dp", "k_max": 8, "n_skip": 44, "interval": 8})
        assert toks2 == ar2
    finally:
        eng.set_decode_kernel("vector")


def test_decode_rows_vs_oracle_70b(gpu70b, slice_model):
    """The decode path at the 70B shape (the vector-ALU projections of
    verify rows, K = 8192 and 28672): after the 64-token prefill, a 3-row
    verify; for each sampled layer the oracle first rebuilds that layer's
    keys and values of the prompt from the GPU's own input rows, then runs
    the verify rows through ``oracle.decode.layer_row`` one by one on the
    GPU's inputs; outputs and the rows' logits within 2e-2."""
    eng = gpu70b["eng"]
    eng.prefill(gpu70b["prompt"])
    pre = np.stack([eng.read_states(r) for r in range(P)])          # [P][L+1][d]
    eng.verify(drafts=[17, 4242])
    z = eng.read_logits(3)
    rows = np.stack([eng.read_states(r) for r in range(3)])         # [3][L+1][d]
    eng.accept()
    st = oracle.DecodeState(slice_model, P + 8)
    for l in SLICES:
        oracle.layer_block(slice_model, l, pre[:, l, :].astype(np.float32), st)
        worst = 0.0
        for i in range(3):
            ho = oracle.decode.layer_row(slice_model, l, rows[i, l, :].astype(np.float32), P + i, st, "full")
            worst = max(worst, float(np.max(np.abs(rows[i, l + 1, :] - ho))))
        print(f"layer {l}: verify rows max-abs {worst:.3e}", flush=True)
        assert worst <= TOL
    for i in range(3):
        zo = slice_model.head(rows[i, SHAPE.n_layers, :].astype(np.float32))
        err = float(np.max(np.abs(z[i] - zo)))
        print(f"verify row {i} logits max-abs {err:.3e}", flush=True)
        assert err <= TOL
