"""Seeded weight and prompt generators (input data only)."""
import numpy as np

from .shapes import ModelShape, tensor_names, tensor_shape

_STD = 0.02
_RESIDUAL_SCALE = 0.1
_OUT_PROJ = ("wo", "w_down")
_NORMS = ("final_norm", "attn_norm", "ffn_norm")


def _torch():
    import torch
    return torch


def make_weights(shape: ModelShape, device="cpu", seed=None, planted_identity=(),
                 head_scale=1.0):
    """Return ``[(name, tensor)]`` in canonical order, on ``device``.

    Matrices are in the shape's dtype (float32 or bfloat16, rounded to nearest
    even from a float32 draw); RMSNorm gains are float32 ones.

    Each tensor ``i`` is drawn from its own torch generator seeded with
    ``seed * 1_000_003 + i``.  The same seed gives different values on CPU and
    GPU (different generator engines); every comparison in this repository
    uses one generated set for both sides.

    ``planted_identity``: layers whose ``wo`` and ``w_down`` are zero, which
    makes them exact identities on the residual stream (a fixture for the
    layer-selection search).  ``head_scale`` multiplies the LM head (a
    fixture that sharpens the output distribution).  Both default to the
    plain recipe.
    """
    torch = _torch()
    seed = shape.weight_seed if seed is None else seed
    dt = torch.float32 if shape.dtype == "f32" else torch.bfloat16
    planted = set(int(x) for x in planted_identity)
    out = []
    for i, name in enumerate(tensor_names(shape)):
        shp = tensor_shape(shape, name)
        base = name.split(".")[-1]
        if base in _NORMS:
            t = torch.ones(shp, dtype=torch.float32, device=device)
        else:
            g = torch.Generator(device=device)
            g.manual_seed(seed * 1_000_003 + i)
            t = torch.randn(shp, generator=g, dtype=torch.float32, device=device)
            scale = _STD
            if base in _OUT_PROJ:
                scale *= _RESIDUAL_SCALE
                if int(name.split(".")[1]) in planted:
                    scale = 0.0
            if base == "lm_head":
                scale *= head_scale
            t.mul_(scale)
        if base not in _NORMS:          # norm gains stay float32 in every config
            t = t.to(dt)
        out.append((name, t.contiguous()))
    return out


def make_prompt(shape: ModelShape, n: int, seed=None) -> np.ndarray:
    """``n`` uniform-random token ids in ``[0, vocab)`` (int32)."""
    seed = shape.prompt_seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(0, shape.vocab, size=n, dtype=np.int64).astype(np.int32)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of raw bf16 bit patterns (uint16/int16) to float32."""
    return (bits.astype(np.uint16).astype(np.uint32) << 16).view(np.float32)


def weights_to_numpy(weights):
    """``{name: float32 ndarray}`` holding exactly the values of ``weights``.

    bf16 tensors are widened exactly; nothing is rounded.
    """
    torch = _torch()
    out = {}
    for name, t in weights:
        t = t.detach().to("cpu")
        # bf16 -> float32 widening is exact (the 16 low bits become zero)
        out[name] = t.to(torch.float32).numpy() if t.dtype == torch.bfloat16 else \
            t.numpy().astype(np.float32, copy=False)
    return out


class LazyF32:
    """Read-only mapping name -> float32 ndarray of a weight list, widened on
    each access (no copy is kept).  For oracle runs on models too large to
    hold in float32 at once."""

    def __init__(self, weights):
        self._w = dict(weights)

    def __getitem__(self, name):
        return weights_to_numpy([(name, self._w[name])])[name]

    def __contains__(self, name):
        return name in self._w

    def keys(self):
        return self._w.keys()
