"""RAT+ inference hot path on AMD MI355X (gfx950).

The compute lives in ``librat.so`` (hand-written HIP kernels behind the C ABI
of ``include/rat.h``); :mod:`.binding` is its argument-marshalling layer and
:mod:`.synth` draws the seeded synthetic workloads.
"""
from .binding import (RAT_DTYPE_BF16, RAT_DTYPE_F32, RAT_ERR_CAPACITY,  # noqa: F401
                      RAT_ERR_HIP, RAT_ERR_INVALID_ARG, RAT_ERR_UNSUPPORTED,
                      RAT_ERR_WORKSPACE, RAT_MAX_HEADS, RAT_OK, RatError,
                      alloc_cache, backward_workspace, decode_workspace, lib,
                      layer_workspace, rat_anchor_rows, rat_layer_prefill,
                      rat_layer_workspace_bytes, rat_prefill_backward,
                      rat_stack_prefill, rat_stack_workspace_bytes, stack_workspace,
                      rat_prefill_backward_workspace_bytes,
                      rat_decode_step, rat_decode_step_noalloc, rat_decode_workspace_bytes,
                      rat_dilated_attn_prefill,
                      rat_dilated_attn_prefill_continue, rat_ring_rows,
                      rat_scan_prefill, rat_scan_prefill_continue,
                      rat_scan_workspace_bytes,
                      rat_status_string, rat_version, scan_workspace,
                      TOPK_BLOCK, TOPK_MAX_K, alloc_topk_history,
                      rat_decode_step_topk, rat_topk_cache_build)

__version__ = "0.1.0"
