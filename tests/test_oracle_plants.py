"""Each planted mistake in the oracle is caught by at least one pin (CPU only).

The oracle source compiles one deliberate error when built with
-DPKV_ORACLE_PLANT=n; the default build has none.
"""
import types

import pytest

import oracle as O
from pins import ATTENTION_PINS, GRAPH_PINS

PLANTS = {
    1: "drops the newest key",
    2: "interleaved instead of contiguous head groups",
    3: "softmax scale dropped",
    4: "page index off by one token",
    5: "K rows read in place of V rows",
}


@pytest.mark.parametrize("plant", sorted(PLANTS), ids=lambda p: PLANTS[p].replace(" ", "_"))
def test_plant_is_caught(plant):
    orc = O.Oracle(plant)
    assert orc.lib.pkv_oracle_plant() == plant
    caught = []
    for pin in ATTENTION_PINS:
        try:
            pin(orc)
        except (AssertionError, O.OracleError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"planted mistake '{PLANTS[plant]}' passed every pin"


def test_clean_build_has_no_plant():
    assert O.Oracle(0).lib.pkv_oracle_plant() == 0


# Planted mistakes in the decode-graph bucket rule (oracle/graph.py), each a
# plausible misreading of the pages' list or of the padding.
def _stop_short(mb):  # the list's end taken as exclusive
    return [b for b in (1, 2, 4, 8) if b <= mb] + list(range(16, mb, 16))


def _strict_choice(mb, batch):
    return next((b for b in O.graph.buckets(mb) if b > batch), -1) if batch >= 1 else -1


def _powers_of_two(mb):
    out, b = [], 1
    while b <= mb:
        out.append(b)
        b *= 2
    return out if out and out[-1] == mb else out + [mb]


def _pad_with_zero_slot(slots, lens, batch, bucket):
    return list(slots[:batch]) + [0] * (bucket - batch), list(lens[:batch]) + [0] * (bucket - batch)


GRAPH_PLANTS = {
    "list_stops_before_the_largest_batch": dict(buckets=_stop_short),
    "strictly_larger_bucket": dict(bucket_for=_strict_choice),
    "powers_of_two_only": dict(buckets=_powers_of_two,
                               bucket_for=lambda mb, b: next(
                                   (x for x in _powers_of_two(mb) if x >= b), -1) if b >= 1 else -1),
    "padding_slot_zero": dict(pad_rows=_pad_with_zero_slot),
}


@pytest.mark.parametrize("name", sorted(GRAPH_PLANTS))
def test_graph_plant_is_caught(name):
    planted = types.SimpleNamespace(buckets=O.graph.buckets, bucket_for=O.graph.bucket_for,
                                    pad_rows=O.graph.pad_rows)
    for k, fn in GRAPH_PLANTS[name].items():
        setattr(planted, k, fn)
    caught = []
    for pin in GRAPH_PINS:
        try:
            pin(planted)
        except AssertionError as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"planted mistake '{name}' passed every pin"


# Planted mistakes in the device-state oracle (oracle/metadata.py).
def _writes_off_by_one(table, writes):
    for row, start, values in writes:
        for i, v in enumerate(values):
            if start + 1 + i < len(table[row]):
                table[row][start + 1 + i] = v
    return table


def _state_ignoring_idx(idx, computed, sched, table, bs, maxb):
    return O.prepare_from_state(list(range(len(idx))), computed, sched, table, bs, maxb)


def _state_dropping_cached(idx, computed, sched, table, bs, maxb):
    return O.prepare_from_state(idx, [0] * len(computed), sched, table, bs, maxb)


META_PLANTS = {
    "write_one_column_late": dict(apply_row_writes=_writes_off_by_one),
    "batch_row_as_state_row": dict(prepare_from_state=_state_ignoring_idx),
    "cached_tokens_dropped": dict(prepare_from_state=_state_dropping_cached),
}


@pytest.mark.parametrize("name", sorted(META_PLANTS))
def test_meta_plant_is_caught(name):
    from pins import META_PINS
    planted = types.SimpleNamespace(apply_row_writes=O.apply_row_writes,
                                    prepare_from_state=O.prepare_from_state,
                                    prepare_prefill=O.prepare_prefill)
    for k, fn in META_PLANTS[name].items():
        setattr(planted, k, fn)
    caught = []
    for pin in META_PINS:
        try:
            pin(planted)
        except AssertionError as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"planted mistake '{name}' passed every pin"
