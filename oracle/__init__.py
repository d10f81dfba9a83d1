"""CPU oracle for the RAT+ hot path (plain C in IEEE double + numpy glue).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP library in ``dilated_sparse_attention_rat_amd``.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py``
against closed forms, brute force and library routines; nothing in it is
"parity unpinned".
"""
from .oracle import (anchor_offsets, attention, attention_rows, backward, build,  # noqa: F401
                     build_cache, decode_step, in_keyset, keyset_size, layer_prefill, lib,
                     num_threads, prefill, round_bf16, scan, set_threads, stack_prefill)
from .topk import (TOPK_BLOCK, block_means, decode_step_topk, keys_topk,  # noqa: F401
                   select_blocks)
