"""MI355X (gfx950) Kimi Delta Attention: chunked prefill and T=1 decode.

The compute runs in ``libkda.so`` (hand-written HIP kernels behind the C ABI
of ``include/kda.h``); this package is its Python binding.  Importing the
package does not load the library; the first call does, and raises if the
library has not been built.
"""
from ._lib import (ANCHOR_DATA, ANCHOR_FIXED, ANCHOR_SPLIT16, GATE_LOG, GATE_LOWER_BOUND, GATE_SOFTPLUS, ROUTE_AUTO,
                   ROUTE_CHUNK, ROUTE_SERIAL, ROUTE_SPLIT, ROUTE_STREAM, FrontEnd, KdaError, Plan, check_prefill_inputs,
                   check_slots, checkpoint_slots, decode, last_error, load, plan, prefill, prefill_chain,
                   prefill_noalloc, NOALLOC_SCRATCH_BYTES,
                   prefill_pool, prefill_prepare, records_size, set_prefill_route, workspace_size)

__all__ = ["prefill", "prefill_noalloc", "NOALLOC_SCRATCH_BYTES", "prefill_pool", "checkpoint_slots", "prefill_prepare", "prefill_chain",
           "records_size", "decode", "plan", "check_prefill_inputs", "check_slots",
           "set_prefill_route", "workspace_size", "last_error",
           "load", "KdaError", "Plan", "ROUTE_AUTO", "ROUTE_SERIAL", "ROUTE_CHUNK", "ROUTE_SPLIT", "ROUTE_STREAM",
           "ANCHOR_FIXED", "ANCHOR_SPLIT16", "ANCHOR_DATA", "FrontEnd", "GATE_LOG", "GATE_LOWER_BOUND",
           "GATE_SOFTPLUS"]
