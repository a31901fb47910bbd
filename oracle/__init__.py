"""fp64 CPU oracle for context-parallel causal attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the bench's CPU-baseline leg, never by the product package.  It shares no
code with the HIP library (``context_attention_cpattn_amd``).

Every function is pinned by ``tests/test_oracle.py`` and
``tests/test_oracle_ring_cache.py`` against brute force on
tiny inputs, torch's fp64 scaled-dot-product attention with an explicit mask,
closed forms and exact identities.
"""
from .attention import attention_rows, full_attention, merge, partial_attention, visible_mask
from .ring import (PASS_KV, PASS_Q, arrival_order, cp_decode, exchange_bytes, pair_visible, ring_attention,
                   schedule, select_order, splitkv_decode)

__all__ = [
    "attention_rows", "full_attention", "merge", "partial_attention", "visible_mask",
    "PASS_KV", "PASS_Q", "arrival_order", "cp_decode", "exchange_bytes", "pair_visible", "ring_attention",
    "schedule", "select_order", "splitkv_decode",
]
