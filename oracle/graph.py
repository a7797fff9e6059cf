"""Oracle of the decode-graph bucket rule -- TEST INFRASTRUCTURE ONLY.

The devpress page ("CUDAGraph优化") and the AIInfraGuide 3.6 page (section 5)
capture one decode graph per batch size in a preset list -- 1, 2, 4, 8 and
every multiple of 16 up to the largest batch -- and run a batch of bs rows on
the smallest listed size that is not below bs, after filling the rows past bs
with slot -1 and context length 0.  Batches above 512 run without a graph.

Reading where the pages are silent: when the largest batch is not a multiple
of 16 it is listed as well, so that every batch up to it has a graph.

Pure Python on purpose: the slow, plain rule the library's bucket choice and
padding are compared with.
"""
from __future__ import annotations

from typing import List, Sequence, Tuple

MAX_GRAPH_BATCH = 512


def buckets(max_batch: int) -> List[int]:
    """The preset batch sizes captured for a largest batch of ``max_batch``."""
    if not 1 <= max_batch <= MAX_GRAPH_BATCH:
        return []
    sizes = [b for b in (1, 2, 4, 8) if b <= max_batch]
    b = 16
    while b <= max_batch:
        sizes.append(b)
        b += 16
    if sizes[-1] != max_batch:
        sizes.append(max_batch)
    return sizes


def bucket_for(max_batch: int, batch: int) -> int:
    """Smallest preset size >= batch; -1 when none (batch < 1 or above the largest)."""
    if batch < 1:
        return -1
    for b in buckets(max_batch):
        if b >= batch:
            return b
    return -1


def pad_rows(slot_mapping: Sequence[int], context_lens: Sequence[int], batch: int,
             bucket: int) -> Tuple[List[int], List[int]]:
    """The step's metadata as the bucket's graph sees it: the first ``batch``
    rows as given, rows batch .. bucket-1 with slot -1 and context length 0."""
    slots = list(slot_mapping[:batch]) + [-1] * (bucket - batch)
    lens = list(context_lens[:batch]) + [0] * (bucket - batch)
    return slots, lens
