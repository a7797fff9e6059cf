"""Oracle copy of the host metadata step -- TEST INFRASTRUCTURE ONLY.

Turns the block manager's per-sequence state into the tensors the attention
step reads, following the two preparation routines of the AIInfraGuide 3.6
page ("ModelRunner、CUDA Graph 与性能基准", section 2):

- prefill: for each sequence with c cached and n scheduled tokens, positions
  c .. c+n-1, cu_seqlens_q grows by n, cu_seqlens_k by c + n, and every new
  token i gets slot block_table[i // block_size] * block_size + i % block_size;
- decode: one token per sequence, context_lens = len(seq) (the stored token
  included), slot = block_table[-1] * block_size + last_block_num_tokens - 1,
  where last_block_num_tokens = len - (num_blocks - 1) * block_size;
- block tables are right-padded with -1 to a common width (same page, and the
  devpress page's parameter list for flash_attn_with_kvcache).

Pure-Python loops on purpose: this is the slow reference the product's native
metadata routine is compared with.
"""
from __future__ import annotations

from typing import List, Sequence


def _table(seqs, max_blocks_per_seq: int) -> List[List[int]]:
    rows = []
    for s in seqs:
        ids = list(s.block_ids)
        if len(ids) > max_blocks_per_seq:
            raise ValueError("sequence owns more blocks than the table width")
        rows.append(ids + [-1] * (max_blocks_per_seq - len(ids)))
    return rows


def prepare_prefill(seqs: Sequence, block_size: int, max_blocks_per_seq: int) -> dict:
    slot_mapping: List[int] = []
    positions: List[int] = []
    cu_q, cu_k = [0], [0]
    for s in seqs:
        c, n = s.num_cached, s.num_new
        if (c + n + block_size - 1) // block_size > len(s.block_ids):
            raise ValueError("sequence has fewer blocks than its tokens need")
        positions.extend(range(c, c + n))
        cu_q.append(cu_q[-1] + n)
        cu_k.append(cu_k[-1] + c + n)
        for i in range(c, c + n):
            block = s.block_ids[i // block_size]
            slot_mapping.append(block * block_size + i % block_size)
    return dict(
        slot_mapping=slot_mapping,
        positions=positions,
        cu_seqlens_q=cu_q,
        cu_seqlens_k=cu_k,
        context_lens=[s.num_cached + s.num_new for s in seqs],
        block_tables=_table(seqs, max_blocks_per_seq),
        max_seqlen_q=max([s.num_new for s in seqs] + [0]),
        max_seqlen_k=max([s.num_cached + s.num_new for s in seqs] + [0]),
    )


def prepare_decode(seqs: Sequence, block_size: int, max_blocks_per_seq: int) -> dict:
    slot_mapping: List[int] = []
    positions: List[int] = []
    context_lens: List[int] = []
    for s in seqs:
        if s.num_new != 1:
            raise ValueError("decode stores exactly one token per sequence")
        length = s.num_cached + 1
        nblk = (length + block_size - 1) // block_size
        if nblk != len(s.block_ids):
            raise ValueError("decode expects exactly the blocks the sequence's tokens need")
        last_block_num_tokens = length - (nblk - 1) * block_size
        positions.append(length - 1)
        context_lens.append(length)
        slot_mapping.append(s.block_ids[-1] * block_size + last_block_num_tokens - 1)
    return dict(
        slot_mapping=slot_mapping,
        positions=positions,
        context_lens=context_lens,
        block_tables=_table(seqs, max_blocks_per_seq),
    )


# ------------------------------------------------------- state kept on the GPU
# docs.vllm.com.cn, "Model Runner V2 设计文档": section 4 (StagedWriteTensor:
# ragged writes staged on the host, applied to a table that stays on the
# device) and section 5 (step inputs derived on the device from per-request
# state).  The oracle applies the writes one after the other and derives the
# step inputs by handing the requests' state to prepare_prefill above.


class _Req:
    """A request as prepare_prefill reads it."""

    def __init__(self, block_ids, num_cached, num_new):
        self.block_ids = tuple(block_ids)
        self.num_cached = num_cached
        self.num_new = num_new


def apply_row_writes(table: List[List[int]], writes) -> List[List[int]]:
    """Each write (row, start, values) overwrites table[row][start:start+len(values)],
    in the order given.  Returns the table (modified in place)."""
    for row, start, values in writes:
        for i, v in enumerate(values):
            table[row][start + i] = v
    return table


def prepare_from_state(idx_mapping, num_computed, num_scheduled, block_table,
                       block_size: int, max_blocks_per_seq: int) -> dict:
    """Step metadata for batch rows b whose request lives in row idx_mapping[b]
    of the persistent state: num_computed[r] cached tokens, num_scheduled[b]
    new ones, block ids block_table[r][0..]."""
    reqs = []
    for b, r in enumerate(idx_mapping):
        c, n = num_computed[r], num_scheduled[b]
        nblk = (c + n + block_size - 1) // block_size
        reqs.append(_Req(block_table[r][:nblk], c, n))
    return prepare_prefill(reqs, block_size, max_blocks_per_seq)
