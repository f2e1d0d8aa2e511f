"""CPU oracle for layer-skip self-speculative decoding -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously-correct numpy implementation of what the decoding path
computes.  It is used only by ``tests/``, by ``__graft_entry__.smoke()`` and by
the ``cpu_baseline`` leg of ``bench.py``.  The product path (the HIP engine in
``layer_skip_self_amd``) never imports it, and it shares no code with the
engine: its only common dependency is the seeded input generator
``lss_synth`` (shapes, weights, prompts -- data only).

Sources (the pages this implements; no equations beyond two are printed there):
  * "CAS-Spec" blog (intelliparadigm.com, article 2260101): section 2.1 (DSIA:
    layer sparsity, early exit, 8-bit activation quantization), 2.2 (three
    virtual draft levels), 3.1 (EMA acceptance predictor), 3.2 (latency model).
  * "CAS-Spec: Cascade Adaptive Self-Speculative Decoding ..." (arXiv
    2510.26843 summary page): abstract (DSIA drafts, DyTC routing by
    acceptance and latency heuristics, lossless acceleration).
  * CLaSp article (news.43b.com.cn/a/479818): section 二 (dynamic layer
    skipping, last accepted token's full hidden states as target), section
    三 (draft -> verify -> layer-optimization workflow, the DP over
    (i layers, j skipped) with cosine similarity, sequence-parallel batching
    of the j-states with a special mask), section 四 (interval, exit threshold).
  * Sampling (``oracle.sampling``): the pages' claim that the method keeps the
    full model's output distribution, read as the standard speculative-
    sampling acceptance rule with a counter-based generator.

Floating point: the oracle computes in float64 by default (``dtype``
argument); the pages fix no precision.  Decisions that turn floating point
into integers *inside the method* (int8 activation codes) are taken in
float32, the precision the GPU kernels take them in.  ``OracleModel(...,
kv_dtype="bf16")`` models a KV cache that keeps keys and values rounded to
bfloat16 (``round_bf16``, from their float32 values); the pages fix no cache
precision either.

Parity status per function is listed in each module header.
"""
from .model import (OracleModel, rms_norm, rope, silu, attend, quantize_row, argmax_first, round_bf16,
                    quantize_weight_rows, w8a8_accumulate, w8a8_project)
from .decode import (DecodeState, layer_block, prefill, forward_row, ar_generate, draft, verify,
                     accept, speculative_generate, batch_generate, Policy, top_b, draft_tree, verify_tree,
                     accept_tree)
from .clasp import clasp_dp, brute_force_skip, forward_with_mask_at_target
from .dytc import (ALPHA, A_INIT, ema_update, fit_latency, predict_latency,
                   plan_cascade, update_cascade, plan_tree, update_tree, expected_tree)
from . import sampling

__all__ = [
    "OracleModel", "rms_norm", "rope", "silu", "attend", "quantize_row", "argmax_first", "round_bf16",
    "quantize_weight_rows", "w8a8_accumulate", "w8a8_project",
    "DecodeState", "layer_block", "prefill", "forward_row", "ar_generate", "draft", "verify", "accept",
    "speculative_generate", "batch_generate", "Policy", "clasp_dp", "brute_force_skip", "top_b", "draft_tree", "verify_tree",
    "accept_tree",
    "forward_with_mask_at_target", "ALPHA", "A_INIT", "ema_update", "fit_latency",
    "predict_latency", "plan_cascade", "update_cascade", "plan_tree", "update_tree", "expected_tree",
    "sampling",
]
