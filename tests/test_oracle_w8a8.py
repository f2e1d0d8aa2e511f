"""Pins of the oracle's W8A8 draft projection (CPU only).

The int8-weight draft widens the pages' 8-bit activation quantization
([CAS blog] 2.1) to the weights: each weight row gets the activation rule
(``quantize_row``), and a projection is the exact integer dot product of the
codes times the two scales.  What fixes the expected values:
  * the vectorised weight quantizer equals the pinned row quantizer row by row;
  * the accumulator equals a pure-integer sum (brute force), also at the
    largest magnitude the 70B down projection can reach;
  * the projection equals the float64 product of the dequantized operands to
    float32 rounding (a swapped or inverted scale fails), and stays within the
    closed-form quantization error bound of the unquantized product;
  * a draft of any quality keeps speculative decoding lossless.
"""
import numpy as np
import pytest

import oracle
from oracle.model import quantize_row, quantize_weight_rows, w8a8_accumulate, w8a8_project


def _bf16(a):
    """Round float32 values to bf16 (nearest even), as float32."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def test_weight_quantizer_equals_the_row_quantizer():
    rng = np.random.default_rng(0)
    W = _bf16(rng.normal(0, 0.02, (37, 96)).astype(np.float32))
    W[5] = 0.0                                   # amax = 0 row
    W[9, 3] = 0.5                                # one large element
    Q, S = quantize_weight_rows(W)
    for n in range(W.shape[0]):
        q, s = quantize_row(W[n])
        assert np.array_equal(Q[n], q) and S[n] == s, n
    assert np.all(Q[5] == 0) and S[5] == 0
    assert Q[9, 3] == 127


def test_accumulator_is_exact():
    rng = np.random.default_rng(1)
    Q = rng.integers(-127, 128, (7, 53)).astype(np.int8)
    q = rng.integers(-127, 128, 53).astype(np.int8)
    ref = [sum(int(Q[n, k]) * int(q[k]) for k in range(53)) for n in range(7)]
    assert w8a8_accumulate(Q, q).tolist() == ref
    assert w8a8_accumulate(Q.astype(np.float32), q).tolist() == ref
    # several 1024-column blocks with every partial sum at the largest magnitude
    K3 = 3000
    Q3 = np.where(np.arange(K3) % 3 == 0, 127, -127).astype(np.int8)[None].repeat(2, 0)
    Q3[1] = 127
    q3 = np.where(np.arange(K3) % 3 == 0, 127, -127).astype(np.int8)
    assert w8a8_accumulate(Q3, q3).tolist() == [127 * 127 * K3, sum(127 * int(v) for v in q3)]
    K = 28672                                    # largest K of the shapes (70B down projection)
    big = np.full((2, K), 127, np.int8)
    big[1] = -127
    acc = w8a8_accumulate(big, np.full(K, 127, np.int8))
    assert acc.tolist() == [127 * 127 * K, -127 * 127 * K]


def test_projection_is_the_dequantized_product():
    rng = np.random.default_rng(2)
    W = _bf16(rng.normal(0, 0.02, (64, 256)).astype(np.float32))
    x = rng.normal(0, 1.0, 256)
    Q, S = quantize_weight_rows(W)
    y = w8a8_project(Q, S, x)
    assert y.dtype == np.float32
    q, sx = quantize_row(x)
    deq = (S.astype(np.float64)[:, None] * Q.astype(np.float64)) @ (float(sx) * q.astype(np.float64))
    assert np.allclose(y, deq, rtol=4 * 2.0**-24, atol=0)
    # closed-form bound against the unquantized product: |w - w^| <= s_n / 2, |x - x^| <= s_x / 2
    exact = W.astype(np.float64) @ x
    xh = float(sx) * q.astype(np.float64)
    bound = float(sx) / 2 * np.abs(W).sum(axis=1) + S.astype(np.float64) / 2 * np.abs(xh).sum()
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-6) + 1e-12)
    # and the bound is not vacuous: the error is a small fraction of the signal
    assert np.max(np.abs(y - exact)) < 0.05 * np.max(np.abs(exact))


def test_zero_activation_gives_zero():
    Q, S = quantize_weight_rows(np.ones((4, 32), np.float32))
    assert np.all(w8a8_project(Q, S, np.zeros(32)) == 0)


G = 32


@pytest.mark.parametrize("pol", [oracle.Policy(K=4, skip=(1,), quant=2), oracle.Policy(K=6, skip=(), quant=2),
                                 oracle.Policy(K=5, skip=(2,), quant=2, tau=0.3)], ids=["skip1", "empty", "tau"])
def test_w8a8_draft_keeps_decoding_lossless(tiny_model, tiny_prompt, pol):
    ar = oracle.ar_generate(tiny_model, tiny_prompt, G)
    toks, recs = oracle.speculative_generate(tiny_model, tiny_prompt, G, pol)
    assert toks == ar
    assert sum(r["n"] for r in recs) > 0


def test_w8a8_draft_differs_from_the_activation_only_draft(tiny_model, tiny_prompt):
    """The weight codes change the draft's logits (otherwise the path would
    silently be the activation-only draft), by about the weight quantization
    error."""
    st1, _, _ = oracle.prefill(tiny_model, tiny_prompt, 64)
    st2, _, _ = oracle.prefill(tiny_model, tiny_prompt, 64)
    z1, _ = oracle.forward_row(tiny_model, st1, st1.t0, st1.p, "draft", [0, 0, 0, 0], 1)
    z2, _ = oracle.forward_row(tiny_model, st2, st2.t0, st2.p, "draft", [0, 0, 0, 0], 2)
    d = np.max(np.abs(z1 - z2))
    assert 1e-5 < d < 0.1 * np.max(np.abs(z1))
