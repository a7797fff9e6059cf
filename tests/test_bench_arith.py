"""The benchmark's work counts (algorithmic bytes of a decode call and of a
store, flops of a causal prefill), checked by enumeration on small plans.

The counts follow the problem statement on the pages: a decode query reads
the K and V rows of every context token through the block table (devpress
"nano-vllm解读", decode with the paged cache), store_kvcache reads each new
row and writes it to its slot (same page, KV-cache write), and a causal
prefill query at position c + i attends keys 0 .. c + i (same page, varlen
prefill).  Each test walks tokens, blocks and (query, key) pairs one at a
time, so a wrong closed form (an off-by-one in the causal count, a missed
term) shows up as a mismatch.
"""
from __future__ import annotations

import pytest

import bench
from workloads import custom_plan, make_plan


def _decode_bytes_by_walk(plan) -> int:
    total = 0
    for s in plan.seqs:
        blocks = set()
        for t in range(s.total):
            total += plan.H_kv * plan.d * 2  # K row of the token, all KV heads
            total += plan.H_kv * plan.d * 2  # V row
            blocks.add(t // plan.block_size)
        total += 4 * len(blocks)  # block-table entries read
        total += 4  # the context length
        total += plan.H_q * plan.d * 2  # q of the sequence
        total += plan.H_q * plan.d * 2  # output of the sequence
    return total


def _store_bytes_by_walk(plan) -> int:
    total = 0
    for s in plan.seqs:
        for _ in range(s.num_new):
            total += 4  # slot
            for _tensor in ("k", "v"):
                total += 2 * plan.row_elems * 2  # read the new row, write it to its slot
    return total


def _prefill_flops_by_walk(plan) -> int:
    pairs = 0
    for s in plan.seqs:
        c = s.num_cached
        for i in range(s.num_new):
            for j in range(c + s.num_new):
                if j <= c + i:
                    pairs += 1
    # q.k and p.v: d multiply-adds each (2 flops), for every query head
    return pairs * plan.H_q * 2 * 2 * plan.d


@pytest.mark.parametrize("specs,bs", [
    ([(0, 1), (6, 1), (15, 1), (32, 1)], 16),
    ([(255, 1), (256, 1), (511, 1), (0, 1), (1000, 1)], 256),
    ([(3, 1)], 1024),
])
def test_decode_bytes(specs, bs):
    plan = custom_plan(specs, bs, H_q=16, H_kv=8, d=128)
    assert bench.decode_bytes(plan) == _decode_bytes_by_walk(plan)


def test_decode_bytes_named_tiny():
    plan = make_plan("tiny_decode")
    assert bench.decode_bytes(plan) == _decode_bytes_by_walk(plan)


def test_decode_bytes_named_subset():
    plan = make_plan("qwen3_decode").subset(list(range(0, 256, 37)))
    assert bench.decode_bytes(plan) == _decode_bytes_by_walk(plan)


@pytest.mark.parametrize("specs", [
    [(0, 1), (6, 1), (15, 1)],
    [(0, 5), (256, 17), (37, 200)],
])
def test_store_bytes(specs):
    plan = custom_plan(specs, 16, H_q=4, H_kv=2, d=64)
    assert bench.store_bytes(plan) == _store_bytes_by_walk(plan)


@pytest.mark.parametrize("specs", [
    [(0, 1)],
    [(0, 7), (16, 1), (5, 33)],
    [(512, 100), (0, 129), (256, 256)],
])
def test_prefill_flops(specs):
    plan = custom_plan(specs, 16, H_q=16, H_kv=8, d=128)
    assert bench.prefill_flops(plan) == _prefill_flops_by_walk(plan)


@pytest.mark.parametrize("c,n", [(0, 0), (0, 1), (0, 130), (7, 1), (256, 19)])
def test_causal_pairs(c, n):
    walked = sum(1 for i in range(n) for j in range(c + n) if j <= c + i)
    assert bench.causal_pairs(c, n) == walked
