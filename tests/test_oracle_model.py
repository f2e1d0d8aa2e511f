"""Pins of the oracle's decoder forward (CPU only).

The oracle is checked against things other than itself: an independent
float64 torch re-expression that uses library attention
(``scaled_dot_product_attention``), complex-multiplication RoPE and library
RMSNorm / SiLU; closed forms of RoPE, attention, RMSNorm and SiLU; and
hand-computed int8 codes (tests/golden/int8_quant.txt).
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.decode import DecodeState, layer_row

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- torch re-expression
def _torch_forward(shape, W, tokens, kv_bf16=False):
    """Full causal forward of ``tokens`` in float64 torch; returns logits [P][V]
    and residual states [L+1][P][d].  kv_bf16: keys (after RoPE) and values
    pass through torch's float32 -> bfloat16 conversion first."""
    d64 = torch.float64
    tw = {k: torch.from_numpy(np.asarray(v, dtype=np.float64)) for k, v in W.items()}
    P = len(tokens)
    Hq, Hkv, hd = shape.n_heads, shape.n_kv_heads, shape.head_dim
    h = tw["embed"][torch.as_tensor(np.asarray(tokens, dtype=np.int64))]
    states = [h]
    # complex rotary factors e^{i * t * theta^(-2i/hd)} for pairs (i, i + hd/2)
    inv = torch.pow(torch.tensor(shape.rope_theta, dtype=d64),
                    -torch.arange(0, hd // 2, dtype=d64) * 2.0 / hd)
    ang = torch.arange(P, dtype=d64)[:, None] * inv[None, :]
    rot = torch.polar(torch.ones_like(ang), ang)          # [P][hd/2]

    def apply_rope(x):                                    # x [P][H][hd]
        xc = torch.complex(x[..., : hd // 2], x[..., hd // 2:])
        y = xc * rot[:, None, :]
        return torch.cat([y.real, y.imag], dim=-1)

    for l in range(shape.n_layers):
        p = f"layers.{l}."
        x = F.rms_norm(h, (shape.d_model,), tw[p + "attn_norm"], eps=shape.rms_eps)
        q = (x @ tw[p + "wq"].T).view(P, Hq, hd)
        k = (x @ tw[p + "wk"].T).view(P, Hkv, hd)
        v = (x @ tw[p + "wv"].T).view(P, Hkv, hd)
        q, k = apply_rope(q), apply_rope(k)
        if kv_bf16:
            k = k.to(torch.float32).to(torch.bfloat16).to(d64)
            v = v.to(torch.float32).to(torch.bfloat16).to(d64)
        rep = Hq // Hkv
        k = k.repeat_interleave(rep, dim=1)
        v = v.repeat_interleave(rep, dim=1)
        o = F.scaled_dot_product_attention(q.transpose(0, 1), k.transpose(0, 1),
                                           v.transpose(0, 1), is_causal=True)
        h = h + o.transpose(0, 1).reshape(P, Hq * hd) @ tw[p + "wo"].T
        x = F.rms_norm(h, (shape.d_model,), tw[p + "ffn_norm"], eps=shape.rms_eps)
        h = h + (F.silu(x @ tw[p + "w_gate"].T) * (x @ tw[p + "w_up"].T)) @ tw[p + "w_down"].T
        states.append(h)
    x = F.rms_norm(h, (shape.d_model,), tw["final_norm"], eps=shape.rms_eps)
    return (x @ tw["lm_head"].T).numpy(), [s.numpy() for s in states]


def test_prefill_matches_torch_reexpression(tiny_shape, tiny_weights_np, tiny_model, tiny_prompt):
    _, z, states = oracle.prefill(tiny_model, tiny_prompt, 64)
    tz, ts = _torch_forward(tiny_shape, tiny_weights_np, tiny_prompt)
    np.testing.assert_allclose(z, tz[-1], rtol=0, atol=1e-9)
    for l in range(tiny_shape.n_layers + 1):
        np.testing.assert_allclose(states[l], ts[l][-1], rtol=0, atol=1e-9)


def test_incremental_decode_matches_full_recompute(tiny_shape, tiny_weights_np, tiny_model, tiny_prompt):
    """Greedy decode one row at a time equals a full causal forward over the
    whole generated sequence, at every generated position."""
    G = 12
    toks = oracle.ar_generate(tiny_model, tiny_prompt, G)
    seq = list(tiny_prompt) + toks[:-1]
    tz, _ = _torch_forward(tiny_shape, tiny_weights_np, seq)
    P = len(tiny_prompt)
    for i in range(G):
        assert int(np.argmax(tz[P - 1 + i])) == toks[i]
    st, _, _ = oracle.prefill(tiny_model, tiny_prompt, 64)
    for i in range(1, G):
        z, _ = oracle.forward_row(tiny_model, st, seq[P - 1 + i], P - 1 + i, "full")
        np.testing.assert_allclose(z, tz[P - 1 + i], rtol=0, atol=1e-9)


def test_round_bf16_matches_torch_bfloat16():
    """round_bf16 is torch's float32 -> bfloat16 conversion (round to
    nearest, ties to even), also on exact ties and from float64 input."""
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(4000) * s for s in (1e-6, 1e-2, 1.0, 1e3)]).astype(np.float32)
    hi = rng.integers(0, 0x7F7F, 2000, dtype=np.uint32) << 16       # finite magnitudes
    ties = (hi | 0x8000).view(np.float32)                 # halfway between two bfloat16 values
    ties = np.concatenate([ties, -ties])
    for v in (x, ties):
        ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float32).numpy()
        assert np.array_equal(oracle.round_bf16(v).view(np.uint32), ref.view(np.uint32))
    x64 = rng.standard_normal(4000)
    ref = torch.from_numpy(x64).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16(x64), ref)


def test_bf16_kv_cache_matches_torch_reexpression(tiny_shape, tiny_weights_np, tiny_prompt):
    """With a bf16 KV cache, prefill and every incremental decode step equal
    the torch re-expression whose keys and values go through torch's
    bfloat16 conversion; the rounding does move the logits."""
    model = oracle.OracleModel(tiny_shape, tiny_weights_np, kv_dtype="bf16")
    G = 10
    toks = oracle.ar_generate(model, tiny_prompt, G)
    seq = list(tiny_prompt) + toks[:-1]
    tz, ts = _torch_forward(tiny_shape, tiny_weights_np, seq, kv_bf16=True)
    P = len(tiny_prompt)
    st, z, states = oracle.prefill(model, tiny_prompt, 64)
    np.testing.assert_allclose(z, tz[P - 1], rtol=0, atol=1e-9)
    for l in range(tiny_shape.n_layers + 1):
        np.testing.assert_allclose(states[l], ts[l][P - 1], rtol=0, atol=1e-9)
    for i in range(1, G):
        z, _ = oracle.forward_row(model, st, seq[P - 1 + i], P - 1 + i, "full")
        np.testing.assert_allclose(z, tz[P - 1 + i], rtol=0, atol=1e-9)
    tz32, _ = _torch_forward(tiny_shape, tiny_weights_np, seq)
    assert np.max(np.abs(tz32 - tz)) > 1e-5


def test_gqa_matches_torch_reexpression():
    """Grouped-query attention (4 q-heads per kv-head) against the library path."""
    import lss_synth
    from dataclasses import replace
    sh = replace(lss_synth.SHAPES["tiny"], name="tiny_gqa", n_heads=8, n_kv_heads=2, head_dim=32,
                 rope_theta=5e5, weight_seed=7)
    W = lss_synth.weights_to_numpy(lss_synth.make_weights(sh))
    m = oracle.OracleModel(sh, W)
    prompt = lss_synth.make_prompt(sh, 20, seed=3)
    _, z, _ = oracle.prefill(m, prompt, 32)
    tz, _ = _torch_forward(sh, W, prompt)
    np.testing.assert_allclose(z, tz[-1], rtol=0, atol=1e-9)


# ---------------------------------------------------------------- closed forms
def test_rope_closed_forms():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 64))
    np.testing.assert_array_equal(oracle.rope(x, 0, 1e4), x)           # angle 0 -> identity
    y = oracle.rope(x, 37, 1e4)
    # each (i, i + hd/2) pair is rotated: its length is unchanged
    n0 = x[:, :32] ** 2 + x[:, 32:] ** 2
    n1 = y[:, :32] ** 2 + y[:, 32:] ** 2
    np.testing.assert_allclose(n1, n0, rtol=1e-12)
    # relative-position property: <R_m q, R_n k> depends only on m - n
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    a = oracle.rope(q[None], 50, 1e4)[0] @ oracle.rope(k[None], 45, 1e4)[0]
    b = oracle.rope(q[None], 5, 1e4)[0] @ oracle.rope(k[None], 0, 1e4)[0]
    assert abs(a - b) < 1e-10
    # pair 0 rotates by exactly pos radians (theta^0 = 1)
    e = np.zeros(64); e[0] = 1.0
    r = oracle.rope(e[None], 2, 1e4)[0]
    assert abs(r[0] - np.cos(2.0)) < 1e-15 and abs(r[32] - np.sin(2.0)) < 1e-15


def test_attention_closed_forms():
    rng = np.random.default_rng(1)
    q = rng.standard_normal(16)
    k1, v1 = rng.standard_normal((1, 16)), rng.standard_normal((1, 16))
    np.testing.assert_allclose(oracle.attend(q, k1, v1), v1[0], rtol=0, atol=0)
    ks = np.repeat(rng.standard_normal((1, 16)), 5, axis=0)             # equal scores
    vs = rng.standard_normal((5, 16))
    np.testing.assert_allclose(oracle.attend(q, ks, vs), vs.mean(axis=0), atol=1e-14)
    # scores scaled by 1/sqrt(hd): two keys with q.k = 0 and sqrt(hd)*ln(3)
    hd = 16
    q = np.zeros(hd); q[0] = 1.0
    ks = np.zeros((2, hd)); ks[1, 0] = np.sqrt(hd) * np.log(3.0)
    vs = np.zeros((2, hd)); vs[0, 1] = 1.0; vs[1, 2] = 1.0
    o = oracle.attend(q, ks, vs)
    assert abs(o[1] - 0.25) < 1e-14 and abs(o[2] - 0.75) < 1e-14


def test_rmsnorm_and_silu_closed_forms():
    rng = np.random.default_rng(2)
    h = rng.standard_normal(256) * 7.0
    x = oracle.rms_norm(h, np.ones(256), 0.0)
    assert abs(np.sqrt(np.mean(x * x)) - 1.0) < 1e-14
    np.testing.assert_allclose(oracle.rms_norm(3.0 * h, np.ones(256), 0.0), x, rtol=1e-14)
    g = rng.standard_normal(256)
    np.testing.assert_allclose(oracle.rms_norm(h, g, 0.0), x * g, rtol=1e-14)
    assert oracle.silu(np.array(0.0)) == 0.0
    t = rng.standard_normal(50)
    np.testing.assert_allclose(oracle.silu(t) - oracle.silu(-t), t, atol=1e-14)   # silu(x)-silu(-x)=x
    assert abs(oracle.silu(np.array(1.0)) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-15


def test_zeroed_output_projections_make_identity_layer(tiny_shape, tiny_weights_np):
    W = dict(tiny_weights_np)
    W["layers.2.wo"] = np.zeros_like(W["layers.2.wo"])
    W["layers.2.w_down"] = np.zeros_like(W["layers.2.w_down"])
    m = oracle.OracleModel(tiny_shape, W)
    st = DecodeState(m, 8)
    h = np.random.default_rng(3).standard_normal(tiny_shape.d_model)
    out = layer_row(m, 2, h, 0, st, "full")
    np.testing.assert_array_equal(out, h)


def test_all_layers_skipped_is_head_of_embedding(tiny_shape, tiny_weights_np, tiny_model):
    st = DecodeState(tiny_model, 8)
    z, states = oracle.forward_row(tiny_model, st, 5, 0, "draft", skip=[1] * tiny_shape.n_layers)
    e = tiny_weights_np["embed"][5].astype(np.float64)
    ref = tiny_weights_np["lm_head"].astype(np.float64) @ (
        e / np.sqrt(np.mean(e * e) + tiny_shape.rms_eps))
    np.testing.assert_allclose(z, ref, rtol=0, atol=1e-12)
    assert all(np.array_equal(s, e) for s in states)


def test_argmax_lowest_index_on_ties():
    assert oracle.argmax_first(np.array([1.0, 3.0, 3.0, 2.0])) == 1
    assert oracle.argmax_first(np.array([-1.0, -1.0])) == 0


# ---------------------------------------------------------------- int8 quantization
def _read_quant_golden():
    cases = []
    with open(os.path.join(GOLDEN, "int8_quant.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            xs, qs, sc = (p.strip() for p in line.split(";"))
            num, den = sc.split("/")
            cases.append(([float(t) for t in xs.split()], [int(t) for t in qs.split()],
                          Fraction(int(num), int(den))))
    return cases


@pytest.mark.parametrize("case", _read_quant_golden())
def test_int8_quant_golden(case):
    xs, qs, scale = case
    q, s = oracle.quantize_row(np.array(xs, dtype=np.float32))
    assert q.tolist() == qs
    assert abs(float(s) - float(scale)) <= 1e-7 * max(1.0, float(scale))


def test_int8_quant_bounds():
    rng = np.random.default_rng(4)
    for _ in range(20):
        x = (rng.standard_normal(777) * rng.uniform(0.01, 50)).astype(np.float32)
        q, s = oracle.quantize_row(x)
        assert q.dtype == np.int8 and np.max(np.abs(q.astype(np.int32))) == 127
        # |x - s*q| <= s/2 (plus float32 slack on the scale)
        err = np.abs(x.astype(np.float64) - float(s) * q.astype(np.float64))
        assert np.all(err <= float(s) * 0.5 * (1 + 1e-5) + 1e-6 * np.abs(x))
        i = int(np.argmax(np.abs(x)))
        assert q[i] == (127 if x[i] > 0 else -127)


def test_float32_oracle_tracks_float64_oracle(tiny_shape, tiny_weights_np, tiny_model, tiny_prompt):
    """The large-shape tests use the oracle in float32 (the same code with
    dtype float32); on the 4-layer model it stays within float32 rounding of
    the float64 oracle pinned above: prefill logits and residual states, a
    decode row, and the greedy tokens of a speculative run (where the float64
    top-1/top-2 gap clears the float32 error)."""
    m32 = oracle.OracleModel(tiny_shape, tiny_weights_np, dtype=np.float32)
    st64, z64, s64 = oracle.prefill(tiny_model, tiny_prompt, 80)
    st32, z32, s32 = oracle.prefill(m32, tiny_prompt, 80)
    assert z32.dtype == np.float32
    scale = float(np.max(np.abs(z64)))
    assert np.max(np.abs(z32 - z64)) <= 1e-5 * scale
    for a, b in zip(s32, s64):
        assert np.max(np.abs(a - b)) <= 1e-5 * max(1.0, float(np.max(np.abs(b))))
    assert st32.t0 == st64.t0
    r64, _ = oracle.forward_row(tiny_model, st64, st64.t0, st64.p, "full")
    r32, _ = oracle.forward_row(m32, st32, st32.t0, st32.p, "full")
    assert np.max(np.abs(r32 - r64)) <= 1e-5 * float(np.max(np.abs(r64)))
    t64, _ = oracle.speculative_generate(tiny_model, tiny_prompt, 24, oracle.Policy(K=3, skip=(1, 2)))
    t32, _ = oracle.speculative_generate(m32, tiny_prompt, 24, oracle.Policy(K=3, skip=(1, 2)))
    assert t32 == t64
