"""Checks that tie the oracle to facts fixed outside it.

Each ``pin_*`` function takes an ``oracle.Oracle`` and raises AssertionError
(or the oracle's own error) if the oracle disagrees with:

- a library routine: torch's scaled_dot_product_attention in float64, with its
  own grouped-query mapping and its own lower-right causal mask, on K/V kept
  contiguous in token order (the unpaged definition);
- an invariance the indirection must have: relabelling physical blocks changes
  nothing;
- closed forms: one key returns its value row; a zero query or identical keys
  return the plain mean of the value rows;
- cross-path identities: prefill of one token equals decode; a prefill split
  into chunks equals the unsplit one; sequences sharing prefix blocks and new
  rows give the same outputs.

They are written so that the planted mistakes the oracle can be built with
(dropped key, wrong head grouping, missing scale, off-by-one page index, K read
as V) each fail at least one of them; ``test_oracle_plants.py`` checks that.
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle as O
from workloads import SeqState, custom_plan, make_tensors

TOL = 1e-12  # float64 oracle against float64 library results


def _store_all(orc, plan, tens):
    """Store every new row of ``plan`` with the oracle; returns its metadata."""
    meta = O.prepare_prefill(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    orc.store(tens.k_cache(), tens.v_cache(), tens.k_new(), tens.v_new(), meta["slot_mapping"])
    return meta


def _contiguous_kv(plan, tens, b):
    """K/V rows of sequence b in token order, straight from the new-row tensors
    (every token of the sequence is new in the plans built here)."""
    starts = [0]
    for s in plan.seqs:
        starts.append(starts[-1] + s.num_new)
    k = tens.k_new()[starts[b]:starts[b + 1]].double()
    v = tens.v_new()[starts[b]:starts[b + 1]].double()
    return k, v  # [L, H_kv, d]


def _sdpa(q, k, v, scale, mask=None):
    """q [nq, H_q, d], k/v [nk, H_kv, d] -> [nq, H_q, d] float64 via torch."""
    o = F.scaled_dot_product_attention(
        q.double().transpose(0, 1).unsqueeze(0),
        k.transpose(0, 1).unsqueeze(0),
        v.transpose(0, 1).unsqueeze(0),
        attn_mask=mask, scale=scale, enable_gqa=True,
    )
    return o.squeeze(0).transpose(0, 1)


def _full_plan(lens, bs, H_q, H_kv, d, seed, extra=3):
    return custom_plan([(0, n) for n in lens], bs, H_q, H_kv, d, seed=seed,
                       extra_blocks=extra, kind="prefill")


GEOMS = [  # (block_size, H_q, H_kv, d)
    (16, 4, 2, 64),
    (16, 8, 2, 64),
    (32, 4, 4, 64),
    (16, 8, 1, 128),
]


def pin_decode_equals_library(orc):
    for gi, (bs, H_q, H_kv, d) in enumerate(GEOMS):
        lens = [1, 5, bs, bs + 1, 3 * bs - 2]
        plan = _full_plan(lens, bs, H_q, H_kv, d, seed=10 + gi)
        tens = make_tensors(plan, "cpu", poison=True)
        _store_all(orc, plan, tens)
        dec = [SeqState(s.block_ids, s.total - 1, 1) for s in plan.seqs]
        meta = O.prepare_decode(dec, bs, plan.max_blocks_per_seq)
        g = torch.Generator().manual_seed(99 + gi)
        q = torch.randn(len(lens), H_q, d, generator=g).to(torch.bfloat16)
        scale = 1.0 / math.sqrt(d)
        out = orc.decode(q, tens.k_cache(), tens.v_cache(), meta["block_tables"],
                         meta["context_lens"], scale)
        assert torch.isfinite(out).all()
        for b in range(len(lens)):
            k, v = _contiguous_kv(plan, tens, b)
            ref = _sdpa(q[b:b + 1], k, v, float(torch.tensor(scale, dtype=torch.float32)))
            err = (out[b] - ref[0]).abs().max().item()
            assert err < TOL, f"decode vs library: seq {b} geom {gi} err {err}"


def pin_prefill_equals_library(orc):
    """Causal prefill over a cached prefix, bottom-right aligned, vs torch."""
    for gi, (bs, H_q, H_kv, d) in enumerate(GEOMS):
        specs = [(0, 7), (bs, 5), (2 * bs + 3, bs + 2), (5, 1), (0, 2 * bs + 1)]
        plan = _full_plan([c + n for c, n in specs], bs, H_q, H_kv, d, seed=20 + gi)
        tens = make_tensors(plan, "cpu", poison=True)
        _store_all(orc, plan, tens)
        view = [SeqState(s.block_ids, c, n) for s, (c, n) in zip(plan.seqs, specs)]
        meta = O.prepare_prefill(view, bs, plan.max_blocks_per_seq)
        g = torch.Generator().manual_seed(7 + gi)
        T = sum(n for _, n in specs)
        q = torch.randn(T, H_q, d, generator=g).to(torch.bfloat16)
        scale = 1.0 / math.sqrt(d)
        out = orc.prefill(q, tens.k_cache(), tens.v_cache(), meta["block_tables"],
                          meta["cu_seqlens_q"], meta["cu_seqlens_k"], scale)
        assert torch.isfinite(out).all()
        at = 0
        for b, (c, n) in enumerate(specs):
            k, v = _contiguous_kv(plan, tens, b)
            mask = causal_lower_right(n, c + n)
            ref = _sdpa(q[at:at + n], k, v, float(torch.tensor(scale, dtype=torch.float32)), mask)
            err = (out[at:at + n] - ref).abs().max().item()
            assert err < TOL, f"prefill vs library: seq {b} geom {gi} err {err}"
            at += n


def _relabel(plan, tens, perm):
    """Same logical content under physical ids perm[p]."""
    pool = torch.empty_like(tens.pool)
    pool[:, :, perm] = tens.pool
    seqs = [SeqState(tuple(int(perm[p]) for p in s.block_ids), s.num_cached, s.num_new)
            for s in plan.seqs]
    return pool, seqs


def pin_permutation_invariance(orc):
    bs, H_q, H_kv, d = 16, 8, 2, 64
    specs = [(0, 3), (40, 9), (16, 16), (70, 1)]
    plan = custom_plan(specs, bs, H_q, H_kv, d, seed=5, extra_blocks=4, kind="prefill")
    tens = make_tensors(plan, "cpu", poison=True)
    meta = _store_all(orc, plan, tens)
    g = torch.Generator().manual_seed(3)
    q = torch.randn(plan.total_new, H_q, d, generator=g).to(torch.bfloat16)
    out = orc.prefill(q, tens.k_cache(), tens.v_cache(), meta["block_tables"],
                      meta["cu_seqlens_q"], meta["cu_seqlens_k"], 0.125)
    perm = torch.randperm(plan.num_blocks, generator=g)
    pool2, seqs2 = _relabel(plan, tens, perm)
    meta2 = O.prepare_prefill(seqs2, bs, plan.max_blocks_per_seq)
    out2 = orc.prefill(q, pool2[0, 0], pool2[1, 0], meta2["block_tables"],
                       meta2["cu_seqlens_q"], meta2["cu_seqlens_k"], 0.125)
    assert torch.equal(out, out2), "relabelling physical blocks changed the output"
    # the relabelled tables really differ
    assert meta["block_tables"] != meta2["block_tables"]


def pin_closed_forms(orc):
    bs, H_q, H_kv, d = 16, 4, 2, 64
    # (a) a sequence of one token returns that token's value row, exactly
    plan = _full_plan([1, 1, 1], bs, H_q, H_kv, d, seed=31)
    tens = make_tensors(plan, "cpu", poison=True)
    _store_all(orc, plan, tens)
    dec = [SeqState(s.block_ids, 0, 1) for s in plan.seqs]
    meta = O.prepare_decode(dec, bs, plan.max_blocks_per_seq)
    q = torch.randn(3, H_q, d).to(torch.bfloat16)
    out = orc.decode(q, tens.k_cache(), tens.v_cache(), meta["block_tables"],
                     meta["context_lens"], 0.125)
    G = H_q // H_kv
    for b in range(3):
        for h in range(H_q):
            assert torch.equal(out[b, h], tens.v_new()[b, h // G].double()), "one key != its value"
    # (b) zero query: uniform weights -> plain mean of the value rows
    # (c) identical keys: uniform weights as well
    lens = [5, 33, 40]
    for identical_keys in (False, True):
        plan = _full_plan(lens, bs, H_q, H_kv, d, seed=32)
        tens = make_tensors(plan, "cpu", poison=True)
        if identical_keys:
            at = 0
            for n in lens:
                tens.k_new()[at:at + n] = tens.k_new()[at:at + 1].clone()
                at += n
        _store_all(orc, plan, tens)
        dec = [SeqState(s.block_ids, s.total - 1, 1) for s in plan.seqs]
        meta = O.prepare_decode(dec, bs, plan.max_blocks_per_seq)
        if identical_keys:
            q = torch.randn(3, H_q, d).to(torch.bfloat16)
        else:
            q = torch.zeros(3, H_q, d, dtype=torch.bfloat16)
        out = orc.decode(q, tens.k_cache(), tens.v_cache(), meta["block_tables"],
                         meta["context_lens"], 0.125)
        for b in range(3):
            _, v = _contiguous_kv(plan, tens, b)
            mean = v.mean(dim=0)  # [H_kv, d]
            for h in range(H_q):
                err = (out[b, h] - mean[h // G]).abs().max().item()
                assert err < TOL, f"uniform-weight case: err {err}"


def pin_prefill_one_equals_decode(orc):
    bs, H_q, H_kv, d = 16, 8, 2, 64
    lens = [1, 9, 16, 17, 50]
    plan = custom_plan([(n - 1, 1) for n in lens], bs, H_q, H_kv, d, seed=41)
    tens = make_tensors(plan, "cpu", poison=True)
    mp = O.prepare_prefill(plan.seqs, bs, plan.max_blocks_per_seq)
    md = O.prepare_decode(plan.seqs, bs, plan.max_blocks_per_seq)
    orc.store(tens.k_cache(), tens.v_cache(), tens.k_new(), tens.v_new(), md["slot_mapping"])
    q = tens.q[0]
    a = orc.decode(q, tens.k_cache(), tens.v_cache(), md["block_tables"], md["context_lens"], 0.125)
    b = orc.prefill(q, tens.k_cache(), tens.v_cache(), mp["block_tables"], mp["cu_seqlens_q"],
                    mp["cu_seqlens_k"], 0.125)
    assert torch.isfinite(a).all()
    assert torch.equal(a, b), "prefill of one token != decode"


def pin_chunked_prefill(orc):
    bs, H_q, H_kv, d = 16, 4, 2, 64
    specs = [(16, 30), (0, 21)]
    plan = custom_plan(specs, bs, H_q, H_kv, d, seed=51, kind="prefill")
    tens = make_tensors(plan, "cpu", poison=True)
    meta = _store_all(orc, plan, tens)
    q = tens.q[0]
    full = orc.prefill(q, tens.k_cache(), tens.v_cache(), meta["block_tables"],
                       meta["cu_seqlens_q"], meta["cu_seqlens_k"], 0.125)
    # first chunk: n1 tokens; second chunk: the rest on top of a longer prefix
    cut = [11, 8]
    first = [SeqState(s.block_ids, c, n1) for s, (c, _), n1 in zip(plan.seqs, specs, cut)]
    second = [SeqState(s.block_ids, c + n1, n - n1) for s, (c, n), n1 in zip(plan.seqs, specs, cut)]
    m1 = O.prepare_prefill(first, bs, plan.max_blocks_per_seq)
    m2 = O.prepare_prefill(second, bs, plan.max_blocks_per_seq)
    rows1, rows2 = [], []
    at = 0
    for (c, n), n1 in zip(specs, cut):
        rows1 += list(range(at, at + n1))
        rows2 += list(range(at + n1, at + n))
        at += n
    o1 = orc.prefill(q[rows1], tens.k_cache(), tens.v_cache(), m1["block_tables"],
                     m1["cu_seqlens_q"], m1["cu_seqlens_k"], 0.125)
    o2 = orc.prefill(q[rows2], tens.k_cache(), tens.v_cache(), m2["block_tables"],
                     m2["cu_seqlens_q"], m2["cu_seqlens_k"], 0.125)
    assert torch.equal(full[rows1], o1) and torch.equal(full[rows2], o2), "chunking changed output"


def pin_shared_prefix(orc):
    bs, H_q, H_kv, d = 16, 4, 2, 64
    specs = [(32, 5), (32, 5), (48, 3)]
    plan = custom_plan(specs, bs, H_q, H_kv, d, seed=61, share_first=(2, 2), kind="prefill")
    assert plan.seqs[0].block_ids[:2] == plan.seqs[1].block_ids[:2]
    tens = make_tensors(plan, "cpu", poison=True)
    tens.kv_new[0, 5:10] = tens.kv_new[0, 0:5]  # identical new rows for seqs 0 and 1
    q = tens.q[0].clone()
    q[5:10] = q[0:5]
    meta = _store_all(orc, plan, tens)
    out = orc.prefill(q, tens.k_cache(), tens.v_cache(), meta["block_tables"],
                      meta["cu_seqlens_q"], meta["cu_seqlens_k"], 0.125)
    assert torch.isfinite(out).all()
    assert torch.equal(out[0:5], out[5:10]), "sequences sharing a prefix disagree"
    assert not torch.equal(out[0:3], out[10:13])


def pin_packed_prefill_equals_library(orc):
    """Varlen prefill over packed K/V (token rows of all sequences stacked, the
    varlen call without a block table), with and without a prefix (nq < nk),
    from row-strided views of one fused QKV buffer, vs torch per sequence."""
    for gi, (_, H_q, H_kv, d) in enumerate(GEOMS):
        specs = [(0, 7), (16, 5), (35, 18), (5, 1), (0, 33), (0, 0)]  # (prefix, new)
        g = torch.Generator().manual_seed(40 + gi)
        nq = [n for _, n in specs]
        nk = [c + n for c, n in specs]
        cu_q = [0]
        cu_k = [0]
        for a, b in zip(nq, nk):
            cu_q.append(cu_q[-1] + a)
            cu_k.append(cu_k[-1] + b)
        # fused rows: q of the new tokens and k/v of all keys, one buffer each
        width = (H_q + 2 * H_kv) * d
        qbuf = torch.randn(cu_q[-1], width, generator=g).to(torch.bfloat16)
        kvbuf = torch.randn(cu_k[-1], width, generator=g).to(torch.bfloat16)
        q = qbuf[:, : H_q * d].view(-1, H_q, d)
        k = kvbuf[:, H_q * d: (H_q + H_kv) * d].view(-1, H_kv, d)
        v = kvbuf[:, (H_q + H_kv) * d:].view(-1, H_kv, d)
        scale = 1.0 / math.sqrt(d)
        out = orc.prefill_packed(q, k, v, cu_q, cu_k, scale)
        assert torch.isfinite(out).all()
        for b in range(len(specs)):
            if nq[b] == 0:
                continue
            mask = causal_lower_right(nq[b], nk[b])
            ref = _sdpa(q[cu_q[b]:cu_q[b + 1]], k[cu_k[b]:cu_k[b + 1]].double(),
                        v[cu_k[b]:cu_k[b + 1]].double(),
                        float(torch.tensor(scale, dtype=torch.float32)), mask)
            err = (out[cu_q[b]:cu_q[b + 1]] - ref).abs().max().item()
            assert err < TOL, f"packed prefill vs library: seq {b} geom {gi} err {err}"


ATTENTION_PINS = [
    pin_decode_equals_library,
    pin_prefill_equals_library,
    pin_permutation_invariance,
    pin_closed_forms,
    pin_prefill_one_equals_decode,
    pin_chunked_prefill,
    pin_shared_prefix,
    pin_packed_prefill_equals_library,
]


# ------------------------------------------------------------ decode-graph buckets

def _graph_fixture():
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "graph_buckets.json")
    with open(path) as f:
        return json.load(f)


def pin_graph_bucket_list(g):
    """The preset list for a largest batch of 512, as the pages' formula gives it."""
    fx = _graph_fixture()
    b = g.buckets(fx["max_batch"])
    assert len(b) == fx["count"], f"{len(b)} buckets for 512, want {fx['count']}"
    assert b[:len(fx["first"])] == fx["first"], b[:8]
    assert b[-len(fx["last"]):] == fx["last"], b[-3:]
    assert g.buckets(0) == [] and g.buckets(513) == []


def pin_graph_bucket_choice(g):
    """The chosen bucket is the smallest listed size not below the batch;
    batches above the largest run eagerly."""
    fx = _graph_fixture()
    for batch, want in fx["choices"]:
        got = g.bucket_for(fx["max_batch"], batch)
        assert got == want, f"batch {batch}: bucket {got}, want {want}"
    for batch in fx["eager"] + [0, -1]:
        assert g.bucket_for(fx["max_batch"], batch) == -1, batch
    # small largest batches: the list holds exactly the powers 1..8 and the
    # multiples of 16 up to it, plus the largest batch itself
    for mb in (1, 2, 3, 5, 8, 9, 15, 16, 17, 40, 100):
        want = sorted({x for x in (1, 2, 4, 8) if x <= mb} | set(range(16, mb + 1, 16)) | {mb})
        assert g.buckets(mb) == want, (mb, g.buckets(mb))
        for batch in range(1, mb + 1):
            got = g.bucket_for(mb, batch)
            assert got >= batch and got in want, (mb, batch, got)
            assert not [x for x in want if batch <= x < got], (mb, batch, got)


def pin_graph_padding(g):
    """Rows past the batch become padding: slot -1 (not stored), length 0."""
    slots, lens = g.pad_rows([40, 7, 1029], [41, 8, 1030], 3, 8)
    assert slots == [40, 7, 1029, -1, -1, -1, -1, -1], slots
    assert lens == [41, 8, 1030, 0, 0, 0, 0, 0], lens
    slots, lens = g.pad_rows([3, 4], [5, 6], 2, 2)
    assert (slots, lens) == ([3, 4], [5, 6])


GRAPH_PINS = [pin_graph_bucket_list, pin_graph_bucket_choice, pin_graph_padding]


# ------------------------------------------------- state kept on the device

def _golden(name):
    import json
    import os
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", name)
    with open(path) as f:
        return json.load(f)


def pin_staged_writes_example(m):
    """The pages' StagedWriteTensor example, on a zero table of its shape."""
    fx = _golden("staged_writes.json")
    R, C = fx["shape"]
    table = [[0] * C for _ in range(R)]
    m.apply_row_writes(table, [tuple(w) for w in fx["writes"]])
    nonzero = sorted((r, c, v) for r, row in enumerate(table) for c, v in enumerate(row) if v)
    assert nonzero == sorted(tuple(e) for e in fx["expected_nonzero"]), nonzero


def pin_staged_writes_disjoint_order(m):
    """Disjoint writes commute; a row not written keeps its contents."""
    g = torch.Generator().manual_seed(21)
    R, C = 12, 40
    writes, used = [], set()
    for _ in range(30):
        r = int(torch.randint(0, R, (1,), generator=g))
        s0 = int(torch.randint(0, C, (1,), generator=g))
        n = int(torch.randint(0, C - s0 + 1, (1,), generator=g))
        cells = {(r, s0 + i) for i in range(n)}
        if cells & used:
            continue
        used |= cells
        writes.append((r, s0, [int(x) for x in torch.randint(-9, 99, (n,), generator=g)]))
    base = [[1000 + 100 * r + c for c in range(C)] for r in range(R)]
    a = m.apply_row_writes([row[:] for row in base], writes)
    b = m.apply_row_writes([row[:] for row in base], list(reversed(writes)))
    assert a == b, "disjoint writes must commute"
    for r in range(R):
        for c in range(C):
            if (r, c) not in used:
                assert a[r][c] == base[r][c], (r, c)


def _state_of(plan, perm=None):
    """Persistent state holding plan's sequences; request b in row perm[b]."""
    B = plan.B
    perm = list(range(B)) if perm is None else perm
    R = B + 2  # two rows no batch entry uses
    computed = [7] * R
    table = [[-3] * (plan.max_blocks_per_seq + 2) for _ in range(R)]
    for b, s in enumerate(plan.seqs):
        r = perm[b]
        computed[r] = s.num_cached
        table[r][:len(s.block_ids)] = list(s.block_ids)
    return perm, computed, [s.num_new for s in plan.seqs], table


def pin_state_equals_host_metadata(m):
    """Metadata from request state equals the pinned host step on the same
    sequences, wherever the requests live in the persistent state."""
    plans = [
        custom_plan([(30, 1), (0, 1), (255, 1), (256, 1)], 16, 4, 2, 64, seed=1, extra_blocks=2),
        custom_plan([(0, 40), (33, 5), (64, 0), (16, 17)], 16, 4, 2, 64, seed=2),
        custom_plan([(512, 100), (512, 3), (0, 9)], 256, 4, 2, 64, seed=3, share_first=(2, 2)),
    ]
    for i, plan in enumerate(plans):
        want = m.prepare_prefill(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
        spread = torch.randperm(plan.B + 2, generator=torch.Generator().manual_seed(i))[:plan.B]
        for perm in (None, list(reversed(range(plan.B))), spread.tolist()):
            idx, computed, sched, table = _state_of(plan, perm)
            got = m.prepare_from_state(idx, computed, sched, table, plan.block_size,
                                       plan.max_blocks_per_seq)
            assert got == want, f"plan {i} perm {perm}: {got} != {want}"


def pin_state_decode_growth(m):
    """The decode block-growth fixture through the state path: the new token's
    slot sits in the sequence's last block, at its last position."""
    fx = _golden("p2_decode_block_growth.json")
    for c in fx["cases"]:
        n, bs = c["num_tokens"], c["block_size"]
        ids = list(range(100, 100 + c["blocks"]))
        got = m.prepare_from_state([1], [0, n - 1], [1], [[-1], ids + [-1]], bs, c["blocks"])
        assert got["slot_mapping"][0] // bs == ids[-1], c
        assert got["slot_mapping"][0] % bs == (n - 1) % bs, c
        assert got["context_lens"] == [n] and got["positions"] == [n - 1], c


META_PINS = [pin_staged_writes_example, pin_staged_writes_disjoint_order,
             pin_state_equals_host_metadata, pin_state_decode_growth]


# ------------------------------------------------------------ Gumbel-max sampling

def pin_philox_known_answers(m):
    """The generator's published known-answer vectors."""
    for v in _golden("philox_kat.json")["vectors"]:
        c = [int(x, 16) for x in v["counter"]]
        k = [int(x, 16) for x in v["key"]]
        got = [int(w[0]) for w in m.philox4x32_10([c[0]], [c[1]], [c[2]], [c[3]], k[0], k[1])]
        assert got == [int(x, 16) for x in v["out"]], (v, [hex(x) for x in got])


def pin_gumbel_moments(m):
    """u stays inside (0, 1); g = -ln(-ln u) has the Gumbel mean (Euler's gamma)
    and variance pi^2 / 6."""
    import numpy as np
    g = []
    for seed in range(8):
        w = m.random_words(seed * 7919 + 1, seed, 1 << 17)
        u = m.uniforms(w)
        assert float(u.min()) > 0.0 and float(u.max()) < 1.0
        g.append(m.gumbel(u).astype(np.float64))
    g = np.concatenate(g)
    n = g.shape[0]
    gamma, var = 0.5772156649015329, math.pi ** 2 / 6
    assert abs(g.mean() - gamma) < 5 * math.sqrt(var / n), g.mean()
    # variance of the sample variance: (mu4 - var^2) / n, Gumbel excess kurtosis 12/5
    assert abs(g.var() - var) < 5 * math.sqrt((3 + 2.4 - 1) * var * var / n), g.var()


def pin_draws_follow_softmax(m):
    """The pages' claim: the argmax of logits / T + g is drawn with probability
    softmax(logits / T).  Chi-square over many offsets of one seed."""
    import numpy as np
    logits = np.array([1.0, 2.0, 0.5, -1.0, 3.0, 0.0], dtype=np.float32)
    N = 12000
    for T in (1.0, 0.6, 2.5):
        toks, _ = m.sample(np.tile(logits, (N, 1)), np.full(N, T, np.float32),
                           np.full(N, 99, np.int64), np.arange(N, dtype=np.int64))
        counts = np.bincount(toks, minlength=logits.shape[0]).astype(np.float64)
        z = logits.astype(np.float64) / T
        p = np.exp(z - z.max())
        p /= p.sum()
        chi2 = float(((counts - N * p) ** 2 / (N * p)).sum())
        assert chi2 < 35.0, (T, chi2, counts.tolist(), (N * p).round(1).tolist())  # 5 dof, p ~ 1e-6


def pin_greedy_and_dominant(m):
    """T <= 0 is the first argmax; a logit far above the rest always wins."""
    import numpy as np
    x = np.array([[0.5, 3.0, -1.0, 3.0, 2.0]], np.float32)
    for T in (0.0, -1.0):
        toks, _ = m.sample(x, [T], [5], [0])
        assert toks.tolist() == [1], toks
    row = np.zeros(100, np.float32)
    row[37] = 60.0
    toks, _ = m.sample(np.tile(row, (50, 1)), np.ones(50, np.float32), np.arange(50), np.arange(50))
    assert toks.tolist() == [37] * 50, toks


SAMPLING_PINS = [pin_philox_known_answers, pin_gumbel_moments, pin_draws_follow_softmax,
                 pin_greedy_and_dominant]
