"""Reference model of the per-batch index.  Test infrastructure.

"Multi-LoRA serving: S-LoRA, Punica and adapter batching" ("How the kernels
work") describes a small per-step index tensor mapping each token to its
adapter slot, passed to both kernels; decode rows are treated one token at a
time (BGMV) and prefill rows in contiguous segments that share an adapter
(SGMV).  The per-row routing with "no adapter" comes from the demo of
"S-LoRA: Serving Thousands of Concurrent Adapters in 2026" (Step 1,
adapter id None).

Readings where the pages leave it open: a request's rows form one segment and
adjacent segments with the same adapter are not merged; slot -1 marks a row
or segment with no adapter; decode rows are grouped by slot with a stable
sort, so within a group rows keep ascending order.
"""
from __future__ import annotations

from typing import Callable, Dict, List, Sequence, Tuple

import numpy as np


def token_slots(row_adapter: Sequence[int], slot_of: Callable[[int], int]) -> np.ndarray:
    """Slot of every row, -1 where the row names no adapter."""
    return np.array([-1 if int(a) < 0 else int(slot_of(int(a))) for a in row_adapter], np.int32)


def segments(lengths: Sequence[int], adapter_ids: Sequence[int],
             slot_of: Callable[[int], int]) -> Tuple[np.ndarray, np.ndarray]:
    """seg_start [S+1] (exclusive prefix sum of the lengths) and seg_slot [S]."""
    seg_start = np.zeros(len(lengths) + 1, np.int32)
    for i, n in enumerate(lengths):
        seg_start[i + 1] = seg_start[i] + int(n)
    seg_slot = np.array([-1 if int(a) < 0 else int(slot_of(int(a))) for a in adapter_ids], np.int32)
    return seg_start, seg_slot


def decode_groups(token_slot: Sequence[int], row_offset: int = 0) -> Dict[int, List[int]]:
    """Rows grouped by slot (rows with slot -1 left out), rows ascending."""
    out: Dict[int, List[int]] = {}
    for t, s in enumerate(token_slot):
        if int(s) >= 0:
            out.setdefault(int(s), []).append(t + row_offset)
    return out
