"""Oracle of the per-step segment plan (integer work, compared bit for bit).

TEST INFRASTRUCTURE ONLY.

Definition, from "LoRA serving, embeddings, rerankers, pooling"
(mlinterviewnotes.com), section "vLLM: preallocated stacked buffers plus a
Punica-style Triton kernel": the metadata is a stable sort of the per-token
slot map plus a sorted unique with counts, rebuilt every forward pass; and
from "mstar.engine.resources.lora.pool" (LoraAddressing): tokens packed in
segment order with CSR-style per-slot offsets over all slots.

Reading used: slot 0 (the zero adapter) takes the place of the -1 base
marker; token_order lists token indices sorted by (slot, index);
slot_indptr[s] is the number of tokens whose slot is below s, so empty slots
have empty segments and slot_indptr[S] = T.
"""
from __future__ import annotations

import numpy as np


def plan(slot_ids, S: int):
    """Return (token_order int32[T], slot_indptr int32[S+1], counts int32[S])."""
    slot_ids = np.asarray(slot_ids, dtype=np.int64)
    if slot_ids.size and (slot_ids.min() < 0 or slot_ids.max() >= S):
        raise ValueError("slot id outside [0, S)")
    token_order = np.argsort(slot_ids, kind="stable").astype(np.int32)
    counts = np.bincount(slot_ids, minlength=S).astype(np.int32)
    indptr = np.zeros(S + 1, np.int32)
    indptr[1:] = np.cumsum(counts)
    return token_order, indptr, counts


def work_list(slot_indptr, rows_per_item: int):
    """Work items (slot, first sorted position, row count) covering every
    segment of a slot >= 1 in ascending slot order, cut into pieces of at
    most ``rows_per_item`` rows. Slot 0's segment is not listed."""
    items = []
    S = len(slot_indptr) - 1
    for s in range(1, S):
        b, e = int(slot_indptr[s]), int(slot_indptr[s + 1])
        for p in range(b, e, rows_per_item):
            items.append((s, p, min(rows_per_item, e - p)))
    return np.array(items, np.int32).reshape(-1, 3)
