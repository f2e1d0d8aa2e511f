"""Seeded synthetic inputs shared by the oracle and the HIP engine.

This module holds only input *data*: model shapes, seeded weights and seeded
prompts.  It contains none of the decoding method's arithmetic (no norm,
attention, projection, sampling or layer-selection code), so that the oracle
under ``oracle/`` and the engine under ``layer_skip_self_amd/`` can both take
their inputs from here without sharing any computation.

Weights follow the recipe the CLaSp article motivates (its section on the
method observes that hidden states change slowly from layer to layer):
every matrix is drawn i.i.d. N(0, 0.02^2); the two residual-branch output
projections (attention output ``wo`` and FFN ``w_down``) are further scaled
by 0.1; RMSNorm gains are 1; the LM head is untied from the embedding.
"""
from .shapes import SHAPES, ModelShape, TENSORS_PER_LAYER, tensor_names
from .gen import make_weights, make_prompt, bf16_bits_to_f32, weights_to_numpy, LazyF32

__all__ = ["SHAPES", "ModelShape", "TENSORS_PER_LAYER", "tensor_names",
           "make_weights", "make_prompt", "bf16_bits_to_f32", "weights_to_numpy", "LazyF32"]
