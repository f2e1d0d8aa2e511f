"""Oracle decoder forward (Llama-style), one layer at a time.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

What it follows:
  * The target model is a LLaMA-family decoder (CLaSp article, section 四:
    LLaMA3 series; CAS-Spec blog, section 2.1: Llama-2 7B).  The pages give no
    layer equations, so the standard Llama block is written out: pre-RMSNorm,
    rotary position embedding (rotate-half pairing), grouped-query softmax
    attention, residual add, pre-RMSNorm, SwiGLU FFN, residual add; final
    RMSNorm and an untied LM head.
  * Dynamic 8-bit activation quantization (CAS-Spec blog, section 2.1, item 3;
    CAS-Spec abstract: "activation quantization"): symmetric per-token int8.

Pins (tests/test_oracle_model.py): an independent float64 torch re-expression
(``scaled_dot_product_attention``, complex-multiply RoPE); closed forms (RoPE at
position 0 is the identity and preserves norms, a single key returns its
value, equal scores average the values, zeroed output projections make a layer
the identity, all-skipped gives head(norm(embedding))); hand-computed int8
codes in tests/golden; incremental decode equals full recompute.  The bf16
KV cache option: ``round_bf16`` equals torch's float32 -> bfloat16
conversion (ties included), and prefill plus every incremental step equal
the torch re-expression with its keys and values converted the same way.
"""
import numpy as np


class OracleModel:
    """Weights (exact float32 values) viewed in the oracle's dtype.

    ``weights``: mapping name -> float32 ndarray, canonical names
    (``embed``, ``final_norm``, ``lm_head``, ``layers.{l}.{wq,...}``).
    ``shape``: an object with the model-shape fields (n_layers, d_model, ...).
    """

    def __init__(self, shape, weights, dtype=np.float64, cache_layers=None, kv_dtype="f32"):
        self.shape = shape
        self.w = weights
        self.dt = np.dtype(dtype)
        # "bf16": the KV cache holds keys and values rounded to bfloat16
        # (``kv``); "f32": unrounded
        if kv_dtype not in ("f32", "bf16"):
            raise ValueError(kv_dtype)
        self.kv_bf16 = kv_dtype == "bf16"
        self.L = shape.n_layers
        self.d = shape.d_model
        self.Hq = shape.n_heads
        self.Hkv = shape.n_kv_heads
        self.hd = shape.head_dim
        self.V = shape.vocab
        self.eps = shape.rms_eps
        self.theta = shape.rope_theta
        if cache_layers is None:
            cache_layers = shape.total_params() * self.dt.itemsize < 2e9
        self._cache = {} if cache_layers else None
        self._w8 = {} if cache_layers else None

    def kv(self, x):
        """The value the KV cache holds for key or value x."""
        return round_bf16(x) if self.kv_bf16 else x

    def _get(self, name):
        if self._cache is not None and name in self._cache:
            return self._cache[name]
        a = np.asarray(self.w[name]).astype(self.dt, copy=False)
        if self._cache is not None:
            self._cache[name] = a
        return a

    def layer(self, l):
        names = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")
        return {n: self._get(f"layers.{l}.{n}") for n in names}

    def layer_w8(self, l):
        """int8 weight copies (codes, row scales) of layer l's projections,
        from the exact float32 weights; cached."""
        key = ("w8", l)
        if self._w8 is not None and key in self._w8:
            return self._w8[key]
        names = ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")
        r = {}
        for n in names:
            Q, S = quantize_weight_rows(np.asarray(self.w[f"layers.{l}.{n}"], np.float32))
            r[n] = (Q.astype(np.float32), S)      # codes kept as exact float32 values
        if self._w8 is not None:
            self._w8[key] = r
        return r

    def embed_row(self, tok):
        if self._cache is not None:
            return self._get("embed")[int(tok)]
        return np.asarray(self.w["embed"][int(tok)]).astype(self.dt)

    def head(self, h):
        """Final RMSNorm + LM head of one residual row -> logits [V]."""
        x = rms_norm(h, self._get("final_norm"), self.eps)
        return self._get("lm_head") @ x

    def head_rows(self, H):
        X = np.stack([rms_norm(h, self._get("final_norm"), self.eps) for h in H])
        return X @ self._get("lm_head").T


def rms_norm(h, g, eps):
    """x = h / sqrt(mean(h^2) + eps) * g  (one row)."""
    return h / np.sqrt(np.mean(h * h) + eps) * g


def rope(x, pos, theta):
    """Rotate-half rotary embedding of ``x`` [n_heads][hd] at position ``pos``.

    Pair (i, i + hd/2) is rotated by angle pos * theta^(-2i/hd); the angles are
    formed in float64 whatever the oracle dtype.
    """
    hd = x.shape[-1]
    half = hd // 2
    i = np.arange(half, dtype=np.float64)
    ang = float(pos) * np.power(float(theta), -2.0 * i / hd)
    c = np.cos(ang).astype(x.dtype)
    s = np.sin(ang).astype(x.dtype)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def silu(x):
    return x / (1.0 + np.exp(-x))


def attend(q, keys, vals):
    """Softmax attention of one query [hd] over keys/vals [n][hd]."""
    s = (keys @ q) / q.dtype.type(np.sqrt(q.shape[-1]))
    s = s - np.max(s)
    p = np.exp(s)
    p = p / np.sum(p)
    return p @ vals


def quantize_row(x):
    """Dynamic symmetric per-token int8 quantization of one activation row.

    amax = max|x|; q = clamp(rint(x * (127 / amax)), -127, 127); scale = amax/127.
    Every decision is taken in float32 (127/amax is one correctly rounded
    float32 division; rint rounds half to even).  amax == 0 gives q = 0 and
    scale 0.  Returns (int8 codes, float32 scale).
    """
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x32))) if x32.size else np.float32(0)
    if amax == 0:
        return np.zeros(x32.shape, np.int8), np.float32(0)
    inv = np.float32(127.0) / amax
    q = np.clip(np.rint(x32 * inv), -127, 127).astype(np.int8)
    return q, np.float32(amax / np.float32(127.0))


def quantize_weight_rows(W):
    """Per-output-row int8 codes of a weight matrix [N][K] (the W8A8 draft's
    weight copy): every row is quantized like an activation row
    (``quantize_row``: float32 decisions, amax / 127 scale, half-even codes),
    written for all rows at once.  Returns (int8 codes [N][K], float32
    scales [N])."""
    W32 = np.asarray(W, dtype=np.float32)
    amax = np.max(np.abs(W32), axis=1).astype(np.float32) if W32.shape[1] else np.zeros(W32.shape[0], np.float32)
    zero = amax == 0
    inv = np.where(zero, np.float32(0), np.float32(127.0) / np.where(zero, np.float32(1), amax)).astype(np.float32)
    Q = np.clip(np.rint(W32 * inv[:, None]), -127, 127).astype(np.int8)
    S = np.where(zero, np.float32(0), amax / np.float32(127.0)).astype(np.float32)
    return Q, S


W8_BLOCK = 1024


def w8a8_accumulate(Q, q):
    """Exact integer dot products sum_k q[k] Q[n][k] (int64).  Q may hold the
    codes as int8 or as their exact float32 values.  Columns are taken in
    blocks of 1024: within a block every product and partial sum is an
    integer of magnitude <= 127^2 * 1024 < 2^24, so a float32 matrix product
    computes the block sum exactly in any order; the block sums are added
    as int64."""
    q32 = np.asarray(q, np.float32)
    acc = np.zeros(Q.shape[0], np.int64)
    for c in range(0, Q.shape[1], W8_BLOCK):
        blk = np.asarray(Q[:, c:c + W8_BLOCK], np.float32) @ q32[c:c + W8_BLOCK]
        acc += np.rint(blk).astype(np.int64)
    return acc


def w8a8_project(Q, S, x):
    """W8A8 projection of one activation row (the int8-weight draft; a
    widening of [CAS blog] 2.1's 8-bit activations to 8-bit weights):
    (q, s_x) = quantize_row(x); y[n] = fl32(fl32(acc_n) * fl32(S[n] * s_x))
    with acc_n the exact integer dot product.  Returns float32 [N]."""
    q, sx = quantize_row(x)
    acc = w8a8_accumulate(Q, q)
    c = (np.asarray(S, np.float32) * np.float32(sx)).astype(np.float32)
    return (acc.astype(np.float32) * c).astype(np.float32)


def round_bf16(x):
    """Nearest bfloat16 value (ties to even) of x taken as float32, in x's
    dtype: bfloat16 keeps the top 16 bits of the float32 encoding."""
    x = np.asarray(x)
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)
    return r.view(np.float32).astype(x.dtype)


def fake_quant(x, dt):
    """The value the draft uses for a quantized input: scale * code."""
    q, s = quantize_row(x)
    return q.astype(dt) * dt.type(s)


def argmax_first(z):
    """Index of the maximum; the lowest index wins ties."""
    return int(np.argmax(z))
