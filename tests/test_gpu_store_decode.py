"""The store fused into the decode call (pkv_store_decode) on the GPU.

It must give what pkv_store of each sequence's new token followed by
pkv_decode gives: the same cache bits and the same output bits (the
arithmetic is the same; only where the new token's row is read from
differs).  The caches start NaN-poisoned outside the stored history, so a
read of the new token's cache row before it is written would show.  One
geometry is also held to the float64 oracle's bar directly.
"""
import pytest
import torch

import paged_kv_cache_110_amd as pkv
from gpu_harness import (assert_bits_equal, assert_close, cpu_copy, device_meta, log,
                         oracle_attention, oracle_meta, oracle_store, scale_of)
from workloads import custom_plan, make_plan, make_tensors

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _fused_vs_split(plan, pad_rows=()):
    split = make_tensors(plan, DEV, poison=True)
    fused = make_tensors(plan, DEV, poison=True)
    meta = pkv.prepare_metadata(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    for i in pad_rows:  # padding rows of a captured batch: slot -1, context 0
        meta["slot_mapping"][i] = -1
        meta["context_lens"][i] = 0
    dm = device_meta(meta, DEV)
    sc = scale_of(plan.d)
    pkv.store(split.k_new(), split.v_new(), split.k_cache(), split.v_cache(), dm["slot_mapping"])
    out_split = pkv.decode(split.q[0], split.k_cache(), split.v_cache(), dm["block_tables"],
                           dm["context_lens"], sc)
    out_fused = pkv.store_decode(fused.q[0], fused.k_new(), fused.v_new(), fused.k_cache(),
                                 fused.v_cache(), dm["block_tables"], dm["context_lens"], sc)
    torch.cuda.synchronize()
    what = f"B={plan.B} G={plan.H_q // plan.H_kv} d={plan.d} bs={plan.block_size}"
    assert_bits_equal(fused.k_cache(), split.k_cache().cpu(), f"k_cache {what}")
    assert_bits_equal(fused.v_cache(), split.v_cache().cpu(), f"v_cache {what}")
    assert_bits_equal(out_fused, out_split.cpu(), f"output {what}")
    return fused, out_fused, meta


GEOMS = [  # (block_size, H_q, H_kv, d)
    (16, 4, 2, 64), (16, 8, 1, 64), (32, 16, 4, 64), (16, 8, 8, 64),
    (256, 16, 8, 128), (16, 4, 4, 128), (64, 32, 8, 128), (256, 64, 8, 128),
    (1024, 16, 2, 128),
]


@pytest.mark.parametrize("geom", GEOMS, ids=lambda g: "bs%d_Hq%d_Hkv%d_d%d" % g)
def test_store_decode_matches_store_then_decode(geom):
    bs, H_q, H_kv, d = geom
    log(f"store_decode geom {geom}")
    g = torch.Generator().manual_seed(7 + sum(geom))
    # the new token alone in its tile (1, 17, bs + 1), at a tile's or block's end (16, bs)
    lens = [1, 2, 16, 17, bs, bs + 1, 3 * bs - 1, 257, 1000, 3001]
    lens += [int(x) for x in torch.randint(1, 3500, (6,), generator=g)]
    plan = custom_plan([(n - 1, 1) for n in lens], bs, H_q, H_kv, d, seed=11 + sum(geom),
                       extra_blocks=5, max_blocks_per_seq=-(-3600 // bs))
    _fused_vs_split(plan, pad_rows=(3,))


@pytest.mark.parametrize("name", ["qwen3_decode", "wide_gqa_decode", "long_decode"])
def test_store_decode_full_size(name):
    """The benchmark workloads (dynamic shares, segments cut over many shares)."""
    log(f"store_decode {name}")
    _fused_vs_split(make_plan(name))


def test_store_decode_against_oracle():
    bs, H_q, H_kv, d = 16, 8, 2, 128
    lens = [1, 5, 16, 33, 200, 777]
    plan = custom_plan([(n - 1, 1) for n in lens], bs, H_q, H_kv, d, seed=91, extra_blocks=3)
    fused, out, meta = _fused_vs_split(plan)
    host = cpu_copy(make_tensors(plan, DEV, poison=True))
    ometa = oracle_meta(plan)
    oracle_store(host, ometa)
    ref = oracle_attention(plan, host, ometa)
    assert_bits_equal(fused.k_cache(), host.k_cache(), "k_cache vs oracle store")
    assert_bits_equal(fused.v_cache(), host.v_cache(), "v_cache vs oracle store")
    assert_close(out, ref, "store_decode vs oracle")


def test_store_decode_clamped_length_stores_nothing():
    """A context length beyond the table's capacity is clamped (as pkv_decode
    clamps it): the new token has no slot, so nothing is stored, and the output
    is pkv_decode's over the clamped length."""
    bs, H_q, H_kv, d = 16, 4, 2, 64
    lens = [20, 33, 48]
    plan = custom_plan([(n - 1, 1) for n in lens], bs, H_q, H_kv, d, seed=5, extra_blocks=2,
                       max_blocks_per_seq=3)
    tens = make_tensors(plan, DEV, poison=False)
    meta = pkv.prepare_metadata(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    dm = device_meta(meta, DEV)
    cl = dm["context_lens"].clone()
    cl[1] = 3 * bs + 5  # beyond 3 blocks of 16
    sc = scale_of(d)
    before_k, before_v = tens.k_cache().clone(), tens.v_cache().clone()
    ref = pkv.decode(tens.q[0], tens.k_cache(), tens.v_cache(), dm["block_tables"], cl, sc)
    out = pkv.store_decode(tens.q[0], tens.k_new(), tens.v_new(), tens.k_cache(), tens.v_cache(),
                           dm["block_tables"], cl, sc)
    torch.cuda.synchronize()
    # rows of sequences 0 and 2 stored, nothing else changed
    slots = meta["slot_mapping"].tolist()
    exp_k, exp_v = before_k.clone(), before_v.clone()
    for b in (0, 2):
        blk, off = divmod(slots[b], bs)
        exp_k[blk, off] = tens.k_new()[b]
        exp_v[blk, off] = tens.v_new()[b]
    assert_bits_equal(tens.k_cache(), exp_k.cpu(), "k_cache with a clamped length")
    assert_bits_equal(tens.v_cache(), exp_v.cpu(), "v_cache with a clamped length")
    # sequence 1 attends over its (clamped) cached rows exactly as pkv_decode does
    assert_bits_equal(out[1], ref[1].cpu(), "output of the clamped sequence")
