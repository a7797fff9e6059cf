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


# Planted mistakes in the sampling oracle (oracle/sampling.py): each variant
# rebuilds the oracle's functions with one plausible error.
def _sampling_variant(noise=None, temper=None, rounds=10, pick=None):
    import numpy as np
    from oracle import sampling as S

    def philox(c0, c1, c2, c3, k0, k1):
        c = [np.asarray(x, dtype=np.uint64) & 0xFFFFFFFF for x in (c0, c1, c2, c3)]
        for _ in range(rounds):
            p0, p1 = c[0] * np.uint64(0xD2511F53), c[2] * np.uint64(0xCD9E8D57)
            c = [(p1 >> np.uint64(32)) ^ c[1] ^ np.uint64(k0), p1 & np.uint64(0xFFFFFFFF),
                 (p0 >> np.uint64(32)) ^ c[3] ^ np.uint64(k1), p0 & np.uint64(0xFFFFFFFF)]
            k0, k1 = (k0 + 0x9E3779B9) & 0xFFFFFFFF, (k1 + 0xBB67AE85) & 0xFFFFFFFF
        return [x.astype(np.uint32) for x in c]

    def words(seed, offset, V):
        q = np.arange((V + 3) // 4, dtype=np.uint64)
        w = philox(q, offset & 0xFFFFFFFF, offset >> 32, 0, seed & 0xFFFFFFFF, seed >> 32)
        return np.stack(w, axis=1).reshape(-1)[:V]

    gumbel = noise or S.gumbel

    def sample(logits, temps, seeds, offsets=None):
        logits = np.asarray(logits, np.float32)
        B = logits.shape[0]
        offsets = np.zeros(B, np.int64) if offsets is None else np.asarray(offsets)
        toks, all_s = np.empty(B, np.int64), []
        for b in range(B):
            T = np.float32(temps[b])
            x = logits[b]
            if T > 0:
                scaled = temper(x, T) if temper else x / T
                s = scaled + gumbel(S.uniforms(words(int(seeds[b]), int(offsets[b]), x.shape[0])))
            else:
                s = x
            toks[b] = (pick or np.argmax)(s)
            all_s.append(s)
        return toks, all_s

    return types.SimpleNamespace(philox4x32_10=philox, random_words=words, uniforms=S.uniforms,
                                 gumbel=gumbel, sample=sample)


def _plain_exponential_noise(u):
    import numpy as np
    return -np.log(u)


SAMPLING_PLANTS = {
    "noise_minus_log_u": dict(noise=_plain_exponential_noise),
    "temperature_multiplies": dict(temper=lambda x, T: x * T),
    "philox_seven_rounds": dict(rounds=7),
    "last_maximum_for_ties": dict(pick=lambda s: len(s) - 1 - int(__import__("numpy").argmax(s[::-1]))),
}


@pytest.mark.parametrize("name", sorted(SAMPLING_PLANTS))
def test_sampling_plant_is_caught(name):
    from pins import SAMPLING_PINS
    planted = _sampling_variant(**SAMPLING_PLANTS[name])
    caught = None
    for pin in SAMPLING_PINS:
        try:
            pin(planted)
        except AssertionError:
            caught = pin.__name__
            break
    assert caught, f"planted mistake '{name}' passed every pin"


def test_sampling_variant_without_plant_passes():
    from pins import SAMPLING_PINS
    clean = _sampling_variant()
    for pin in SAMPLING_PINS:
        pin(clean)
