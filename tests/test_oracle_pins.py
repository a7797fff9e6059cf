"""The oracle against what the pages and the mathematics fix (CPU only)."""
import json
import math
import os

import pytest
import torch

import oracle as O
from pins import ATTENTION_PINS, GRAPH_PINS, META_PINS, SAMPLING_PINS
from workloads import SeqState, custom_plan, make_plan, make_tensors, NAN_BF16_BITS

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="module")
def orc():
    return O.Oracle(0)


# ---------------------------------------------------------------- metadata


def test_p1_logical_mapping_fixture():
    fx = _golden("p1_logical_mapping.json")
    seqs = [SeqState(tuple(s["block_ids"]), 0, s["num_tokens"]) for s in fx["sequences"]]
    meta = O.prepare_prefill(seqs, fx["block_size"], max_blocks_per_seq=2)
    start = {}
    at = 0
    for s in fx["sequences"]:
        start[s["name"]] = at
        at += s["num_tokens"]
    for e in fx["expected_slots"]:
        assert meta["slot_mapping"][start[e["seq"]] + e["token"]] == e["slot"]
    assert meta["block_tables"] == [[0, 1], [2, -1]]


def test_p2_decode_block_growth_fixture():
    fx = _golden("p2_decode_block_growth.json")
    for c in fx["cases"]:
        n, bs = c["num_tokens"], c["block_size"]
        ids = tuple(range(100, 100 + c["blocks"]))
        meta = O.prepare_decode([SeqState(ids, n - 1, 1)], bs, c["blocks"])
        slot = meta["slot_mapping"][0]
        assert slot // bs == ids[-1], "the new token must land in the last block"
        assert slot % bs == c["offset"]
        assert (slot % bs == 0) == c["new_block"]
        # one block fewer is not enough, one more is rejected by the decode form
        with pytest.raises(ValueError):
            O.prepare_decode([SeqState(ids[:-1], n - 1, 1)], bs, c["blocks"])


def test_p3_decode_slot_fixture():
    fx = _golden("p3_decode_slot.json")
    for c in fx["cases"]:
        seq = SeqState(tuple(c["block_ids"]), c["num_tokens"] - 1, 1)
        meta = O.prepare_decode([seq], c["block_size"], len(c["block_ids"]))
        assert meta["slot_mapping"] == [c["slot"]]
        assert meta["context_lens"] == [c["context_len"]]
        assert meta["positions"] == [c["num_tokens"] - 1]


@pytest.mark.parametrize("name", ["tiny_decode", "qwen3_decode", "full_step"])
def test_decode_form_equals_general_form(name):
    """The decode slot form and the per-token prefill loop agree at n = 1."""
    plan = make_plan(name)
    md = O.prepare_decode(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    mp = O.prepare_prefill(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    assert md["slot_mapping"] == mp["slot_mapping"]
    assert md["context_lens"] == mp["context_lens"]
    assert md["block_tables"] == mp["block_tables"]
    assert mp["cu_seqlens_q"] == list(range(plan.B + 1))


def test_prefill_metadata_invariants():
    plan = make_plan("prefix_prefill")
    m = O.prepare_prefill(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    bs = plan.block_size
    slots = m["slot_mapping"]
    assert len(slots) == len(set(slots)) == plan.total_new
    assert all(0 <= s < plan.num_blocks * bs for s in slots)
    for b, s in enumerate(plan.seqs):
        assert m["cu_seqlens_q"][b + 1] - m["cu_seqlens_q"][b] == s.num_new
        assert m["cu_seqlens_k"][b + 1] - m["cu_seqlens_k"][b] == s.num_cached + s.num_new
        row = m["block_tables"][b]
        assert row[: len(s.block_ids)] == list(s.block_ids)
        assert all(x == -1 for x in row[len(s.block_ids):])
    # new tokens never land in a shared prefix block
    shared = set(plan.seqs[0].block_ids[:8])
    assert not any(s // bs in shared for s in slots)
    assert m["max_seqlen_q"] == max(s.num_new for s in plan.seqs)


def test_workload_shapes_match_descriptions():
    t = make_plan("tiny_decode")
    assert [s.total for s in t.seqs] == [1, 7, 16, 33]
    assert [len(s.block_ids) for s in t.seqs] == [1, 1, 1, 3]
    assert t.num_blocks == 32 and t.max_blocks_per_seq == 3
    q = make_plan("qwen3_decode")
    assert q.B == 256 and all(128 <= n <= 2048 for n in q.lens())
    assert q.num_blocks == sum(len(s.block_ids) for s in q.seqs)
    ids = [b for s in q.seqs for b in s.block_ids]
    assert sorted(ids) == list(range(q.num_blocks))
    lg = make_plan("long_decode")
    assert all(8192 <= n <= 32768 for n in lg.lens())
    p = make_plan("prefix_prefill")
    assert all(s.num_cached % 256 == 0 and s.num_cached <= 4096 for s in p.seqs)
    assert all(s.num_cached >= 8 * 256 for s in p.seqs[:4])
    assert len({s.block_ids[:8] for s in p.seqs[:4]}) == 1
    assert all(128 <= s.num_new <= 2048 for s in p.seqs)
    f = make_plan("full_step")
    assert f.B == 512 and f.layers == 28
    assert all(16 <= n <= 16384 for n in f.lens())


# ------------------------------------------------------------------- store


def test_store_layout_and_skip(orc):
    bs, H_q, H_kv, d = 16, 4, 2, 64
    plan = custom_plan([(0, 20), (5, 9), (31, 1)], bs, H_q, H_kv, d, seed=2, extra_blocks=2,
                       kind="prefill")
    tens = make_tensors(plan, "cpu", poison=True)
    meta = O.prepare_prefill(plan.seqs, bs, plan.max_blocks_per_seq)
    slots = list(meta["slot_mapping"])
    skipped = {3, 17, 25}
    for i in skipped:
        slots[i] = -1
    before_k = tens.k_cache().clone()
    before_v = tens.v_cache().clone()
    orc.store(tens.k_cache(), tens.v_cache(), tens.k_new(), tens.v_new(), slots)
    kb = tens.k_cache().view(torch.int16)
    vb = tens.v_cache().view(torch.int16)
    written = torch.zeros(plan.num_blocks, bs, dtype=torch.bool)
    for i, s in enumerate(slots):
        if s == -1:
            continue
        blk, off = divmod(s, bs)
        written[blk, off] = True
        # [num_blocks, block_size, H_kv, d] indexing: row `off` of block `blk`
        assert torch.equal(kb[blk, off], tens.k_new()[i].contiguous().view(torch.int16))
        assert torch.equal(vb[blk, off], tens.v_new()[i].contiguous().view(torch.int16))
    # every other row keeps its exact bits (NaN poison included)
    assert torch.equal(kb[~written], before_k.view(torch.int16)[~written])
    assert torch.equal(vb[~written], before_v.view(torch.int16)[~written])
    # skipped tokens' rows still hold the poison pattern
    for i in skipped:
        blk, off = divmod(meta["slot_mapping"][i], bs)
        assert (kb[blk, off] == NAN_BF16_BITS).all()


def test_store_rejects_bad_slots(orc):
    bs, H_kv, d = 16, 2, 64
    plan = custom_plan([(0, 4)], bs, 2, H_kv, d, seed=3, kind="prefill")
    tens = make_tensors(plan, "cpu", poison=True)
    with pytest.raises(O.OracleError) as e:
        orc.store(tens.k_cache(), tens.v_cache(), tens.k_new(), tens.v_new(), [0, 1, 16, 2])
    assert e.value.code == 2
    with pytest.raises(O.OracleError) as e:
        orc.store(tens.k_cache(), tens.v_cache(), tens.k_new(), tens.v_new(), [0, 1, 1, 2])
    assert e.value.code == 3
    with pytest.raises(O.OracleError) as e:
        orc.store(tens.k_cache(), tens.v_cache(), tens.k_new(), tens.v_new(), [0, -2, 1, 2])
    assert e.value.code == 2


def test_attention_rejects_bad_tables(orc):
    bs, H_q, H_kv, d = 16, 2, 1, 64
    plan = custom_plan([(20, 1)], bs, H_q, H_kv, d, seed=4)
    tens = make_tensors(plan, "cpu", poison=False)
    q = tens.q[0]
    with pytest.raises(O.OracleError) as e:  # padding id read for key 16..20
        orc.decode(q, tens.k_cache(), tens.v_cache(), [[plan.seqs[0].block_ids[0], -1]], [21], 0.125)
    assert e.value.code == 4
    with pytest.raises(O.OracleError) as e:  # context beyond the table width
        orc.decode(q, tens.k_cache(), tens.v_cache(), [list(plan.seqs[0].block_ids)], [33], 0.125)
    assert e.value.code == 5


# --------------------------------------------------------------- attention


@pytest.mark.parametrize("pin", ATTENTION_PINS, ids=lambda f: f.__name__)
def test_attention_pin(orc, pin):
    pin(orc)


def test_zero_length_gives_zero_row(orc):
    bs, H_q, H_kv, d = 16, 4, 2, 64
    plan = custom_plan([(4, 1)], bs, H_q, H_kv, d, seed=8)
    tens = make_tensors(plan, "cpu", poison=True)
    out = orc.decode(tens.q[0], tens.k_cache(), tens.v_cache(), [list(plan.seqs[0].block_ids)],
                     [0], 0.125)
    assert torch.equal(out, torch.zeros_like(out))


def test_poisoned_tiny_config_is_finite(orc):
    plan = make_plan("tiny_decode")
    tens = make_tensors(plan, "cpu", poison=True)
    meta = O.prepare_decode(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    orc.store(tens.k_cache(), tens.v_cache(), tens.k_new(), tens.v_new(), meta["slot_mapping"])
    out = orc.decode(tens.q[0], tens.k_cache(), tens.v_cache(), meta["block_tables"],
                     meta["context_lens"], 1.0 / math.sqrt(plan.d))
    assert torch.isfinite(out).all()
    # context length 1 (sequence 0): the output is the stored value row
    G = plan.H_q // plan.H_kv
    for h in range(plan.H_q):
        assert torch.equal(out[0, h], tens.v_new()[0, h // G].double())


# ------------------------------------------------------------ decode-graph buckets


@pytest.mark.parametrize("pin", GRAPH_PINS, ids=lambda p: p.__name__)
def test_graph_bucket_oracle(pin):
    pin(O.graph)


# ------------------------------------------------- state kept on the device


@pytest.mark.parametrize("pin", META_PINS, ids=lambda p: p.__name__)
def test_device_state_oracle(pin):
    pin(O)


# ------------------------------------------------------------ Gumbel-max sampling


@pytest.mark.parametrize("pin", SAMPLING_PINS, ids=lambda p: p.__name__)
def test_sampling_oracle(pin):
    from oracle import sampling
    pin(sampling)
