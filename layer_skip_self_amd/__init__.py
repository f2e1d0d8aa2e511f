"""MI355X (gfx950) engine for layer-skip self-speculative greedy decoding.

The compute runs in ``liblss.so`` (hand-written HIP kernels behind the C ABI
of ``include/lss.h``); this package only marshals arguments.  Importing it
does not load the library; the first engine call does, and fails loudly if
it has not been built.
"""
from .engine import (Engine, LssError, make_config, workspace_bytes, router_plan, router_update,
                     router_plan_tree, router_update_tree, latency_fit, quantize_rows, make_policy)

__all__ = ["Engine", "LssError", "make_config", "workspace_bytes", "router_plan", "router_update",
           "router_plan_tree", "router_update_tree", "latency_fit", "quantize_rows", "make_policy"]
