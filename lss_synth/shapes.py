"""Model shapes of the synthetic workloads (Llama-style decoders).

The shapes are the public Llama-2-7B / Llama-3-8B / Llama-3-70B layer shapes
plus a tiny 4-layer model; the pages evaluate on LLaMA-family models (CLaSp
article, experiments section) and CAS-Spec quotes a Llama-2 7B table.
"""
from dataclasses import dataclass


@dataclass(frozen=True)
class ModelShape:
    name: str
    n_layers: int
    d_model: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_dim: int
    vocab: int
    rope_theta: float
    dtype: str              # "f32" or "bf16" (storage of weights and KV cache)
    rms_eps: float = 1e-5
    weight_seed: int = 0
    prompt_seed: int = 0

    @property
    def q_dim(self) -> int:
        return self.n_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    def layer_params(self) -> int:
        d, f = self.d_model, self.ffn_dim
        return d * (self.q_dim + 2 * self.kv_dim) + self.q_dim * d + 3 * d * f + 2 * d

    def total_params(self) -> int:
        return self.n_layers * self.layer_params() + 2 * self.vocab * self.d_model + self.d_model


SHAPES = {
    # 4 layers, d 256, 4 MHA heads of 64, SwiGLU 688, vocab 1024, fp32.
    "tiny": ModelShape("tiny", 4, 256, 4, 4, 64, 688, 1024, 1e4, "f32",
                       weight_seed=1, prompt_seed=101),
    # Small bf16 model for fast edge cases of the bf16 decode kernels: 3 L,
    # d 320, 5 q heads / 1 kv head of 64 (GQA 5), SwiGLU 864, vocab 1008.  Its
    # projection depths (320, 864) are not whole numbers of 128-element
    # pieces, and some waves of a decode launch get no piece of K at all.
    "small_bf16": ModelShape("small_bf16", 3, 320, 5, 1, 64, 864, 1008, 1e4, "bf16",
                             weight_seed=11, prompt_seed=111),
    # Medium float32 model for the float32 decode kernels at real depths: 2 L,
    # d 1024, 8 q / 2 kv heads of 128 (GQA 4), SwiGLU 5632, vocab 4096.  Its
    # FFN depth is 22 chunks of 1 KB of float32 weights, so the down
    # projection's waves take 3 or 2 chunks each.
    "medium_f32": ModelShape("medium_f32", 2, 1024, 8, 2, 128, 5632, 4096, 1e4, "f32",
                             weight_seed=13, prompt_seed=113),
    # Wide float32 model, one layer: d 3072 (12 chunks of 1 KB: two chunk
    # registers per wave) and FFN 14336 (56 chunks: eight, at most 2 rows per
    # launch) for the remaining float32 GEMV variants.
    "wide_f32": ModelShape("wide_f32", 1, 3072, 8, 2, 128, 14336, 4096, 1e4, "f32",
                           weight_seed=17, prompt_seed=117),
    # Llama-2-7B shape: 32 L, d 4096, 32 MHA heads, FFN 11008, vocab 32000.
    "llama2_7b": ModelShape("llama2_7b", 32, 4096, 32, 32, 128, 11008, 32000, 1e4, "bf16",
                            weight_seed=2, prompt_seed=102),
    # Llama-3-8B shape: 32 L, d 4096, 32 q / 8 kv heads, FFN 14336, vocab 128256.
    "llama3_8b": ModelShape("llama3_8b", 32, 4096, 32, 8, 128, 14336, 128256, 5e5, "bf16",
                            weight_seed=3, prompt_seed=103),
    # Llama-3-70B shape: 80 L, d 8192, 64 q / 8 kv heads, FFN 28672, vocab 128256.
    "llama3_70b": ModelShape("llama3_70b", 80, 8192, 64, 8, 128, 28672, 128256, 5e5, "bf16",
                             weight_seed=5, prompt_seed=107),
}

# Canonical tensor order (also the order the C-ABI expects):
#   embed [V][d], final_norm [d], lm_head [V][d], then per layer:
#   attn_norm [d], wq [Hq*hd][d], wk [Hkv*hd][d], wv [Hkv*hd][d], wo [d][Hq*hd],
#   ffn_norm [d], w_gate [F][d], w_up [F][d], w_down [d][F]
LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")
TENSORS_PER_LAYER = len(LAYER_TENSORS)
GLOBAL_TENSORS = ("embed", "final_norm", "lm_head")


def tensor_names(shape: ModelShape):
    names = list(GLOBAL_TENSORS)
    for layer in range(shape.n_layers):
        names += [f"layers.{layer}.{t}" for t in LAYER_TENSORS]
    return names


def tensor_shape(shape: ModelShape, name: str):
    d, f, v = shape.d_model, shape.ffn_dim, shape.vocab
    base = name.split(".")[-1]
    return {
        "embed": (v, d), "final_norm": (d,), "lm_head": (v, d),
        "attn_norm": (d,), "wq": (shape.q_dim, d), "wk": (shape.kv_dim, d),
        "wv": (shape.kv_dim, d), "wo": (d, shape.q_dim), "ffn_norm": (d,),
        "w_gate": (f, d), "w_up": (f, d), "w_down": (d, f),
    }[base]
