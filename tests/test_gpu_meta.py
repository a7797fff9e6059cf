"""Step metadata built on the device and staged block-table writes
(pkv_prepare_metadata_device, pkv_apply_row_writes), on the GPU: every output
bit-exact against the oracle (oracle/metadata.py), and the device metadata
driving the store and decode kernels to the same bits as the host metadata."""
import pytest
import torch

import oracle as O
import paged_kv_cache_110_amd as pkv
from gpu_harness import assert_close, cpu_copy, log, oracle_attention, oracle_meta, scale_of
from workloads import custom_plan, make_tensors

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _disjoint_writes(g, R, C, count):
    writes, used = [], set()
    while len(writes) < count:
        r = int(torch.randint(0, R, (1,), generator=g))
        s0 = int(torch.randint(0, C, (1,), generator=g))
        n = int(torch.randint(0, min(C - s0, 40) + 1, (1,), generator=g))
        cells = {(r, s0 + i) for i in range(n)}
        if cells & used:
            continue
        used |= cells
        writes.append((r, s0, [int(x) for x in torch.randint(-5, 1 << 30, (n,), generator=g)]))
    return writes


@pytest.mark.parametrize("strided", [False, True])
def test_staged_writes_match_oracle(strided):
    g = torch.Generator().manual_seed(31 + strided)
    R, C = 300, 128
    init = torch.randint(-1, 5000, (R, C + 32 if strided else C), generator=g, dtype=torch.int32)
    big = init.to(DEV)
    table = big[:, :C] if strided else big
    host = [row[:C] for row in init.tolist()]
    st = pkv.StagedWrites(table)
    for rnd in range(3):
        writes = _disjoint_writes(g, R, C, 200 if rnd else 1)
        writes.append((R - 1, 0, list(range(C))))  # a whole row
        writes.append((5, C - 1, [424242]))        # the last column
        writes = [w for i, w in enumerate(writes)
                  if not any(w[0] == v[0] and max(w[1], v[1]) < min(w[1] + len(w[2]), v[1] + len(v[2]))
                             for v in writes[:i])]
        log(f"staged writes round {rnd}: {len(writes)} writes, {sum(len(w[2]) for w in writes)} values")
        for row, start, values in writes:
            st.stage_write(row, start, values)
        st.apply()
        torch.cuda.synchronize()
        O.apply_row_writes(host, writes)
        assert table.cpu().tolist() == host, f"round {rnd}"
        if strided:  # columns past the view are never written
            assert torch.equal(big[:, C:].cpu(), init[:, C:])


def _state_case(g, B, R, width, bs, cmax, nmax, zero_every=0):
    idx = torch.randperm(R, generator=g)[:B].to(torch.int32)
    computed = torch.randint(0, cmax + 1, (R,), generator=g, dtype=torch.int32)
    sched = torch.randint(1 if nmax else 0, nmax + 1, (B,), generator=g, dtype=torch.int32)
    if zero_every:
        sched[::zero_every] = 0
    need = [-(-(int(computed[int(r)]) + int(n)) // bs) for r, n in zip(idx, sched)]
    maxb = max(need + [1])
    assert maxb <= width
    table = torch.randint(0, 1 << 20, (R, width), generator=g, dtype=torch.int32)
    return idx, computed, sched, table, maxb


STATE_CASES = {  # name: (B, R, width, bs, max cached, max new, zero every)
    "decode_B256": (256, 300, 140, 16, 2047, 1, 0),
    "prefill_B16": (16, 40, 25, 256, 4096, 2048, 0),
    "mixed_zero_rows": (100, 120, 40, 64, 1500, 37, 3),
    "B1": (1, 1, 8, 16, 100, 5, 0),
    "B4096": (4096, 4200, 4, 256, 700, 1, 0),
}


@pytest.mark.parametrize("name", sorted(STATE_CASES))
def test_device_metadata_matches_oracle(name):
    B, R, width, bs, cmax, nmax, zero_every = STATE_CASES[name]
    g = torch.Generator().manual_seed(len(name) * 7 + B)
    idx, computed, sched, table, maxb = _state_case(g, B, R, width, bs, cmax, nmax, zero_every)
    want = O.prepare_from_state(idx.tolist(), computed.tolist(), sched.tolist(), table.tolist(), bs,
                                maxb)
    total = want["cu_seqlens_q"][-1]
    log(f"device metadata {name}: B={B}, {total} new tokens, table [{R}, {width}], maxb {maxb}")
    for cap in (total, total + 13, max(total // 2, 1)):
        got = pkv.prepare_metadata_device(idx.to(DEV), computed.to(DEV), sched.to(DEV),
                                          table.to(DEV), bs, maxb, cap)
        torch.cuda.synchronize()
        rows = min(total, cap)
        assert got["cu_seqlens_q"].cpu().tolist() == want["cu_seqlens_q"]
        assert got["cu_seqlens_k"].cpu().tolist() == want["cu_seqlens_k"]
        assert got["context_lens"][:B].cpu().tolist() == want["context_lens"]
        assert got["slot_mapping"][:rows].cpu().tolist() == want["slot_mapping"][:rows]
        assert got["positions"][:rows].cpu().tolist() == want["positions"][:rows]
        assert got["block_tables"].cpu().tolist() == want["block_tables"]
        assert got["max_seqlens"].cpu().tolist() == [want["max_seqlen_q"], want["max_seqlen_k"]]


def test_device_metadata_empty_batch():
    z = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = pkv.prepare_metadata_device(None, z, z[:0], torch.zeros(1, 4, dtype=torch.int32, device=DEV),
                                      16, 4, 0, positions=False, block_tables=False)
    torch.cuda.synchronize()
    assert got["cu_seqlens_q"].cpu().tolist() == [0] and got["cu_seqlens_k"].cpu().tolist() == [0]
    assert got["max_seqlens"].cpu().tolist() == [0, 0]


def test_device_metadata_drives_store_and_decode():
    """Block tables grown by staged writes, metadata built on the device, then
    store + decode: the same bits as the host metadata path, and the oracle's
    attention within the bar."""
    g = torch.Generator().manual_seed(77)
    lens = [int(x) for x in torch.randint(1, 700, (64,), generator=g)]
    plan = custom_plan([(n - 1, 1) for n in lens], 16, 16, 8, 128, seed=77, extra_blocks=5)
    maxb = plan.max_blocks_per_seq
    tens_a = make_tensors(plan, DEV, poison=True)
    tens_b = make_tensors(plan, DEV, poison=True)
    host = cpu_copy(tens_a)
    B, R = plan.B, plan.B + 9
    rows = torch.randperm(R, generator=g)[:B]
    # persistent state: each request's block ids arrive as a few staged writes
    table = torch.full((R, maxb + 3), -1, dtype=torch.int32, device=DEV)
    st = pkv.StagedWrites(table)
    for b, s in enumerate(plan.seqs):
        ids = list(s.block_ids)
        cut = len(ids) // 2
        st.stage_write(int(rows[b]), 0, ids[:cut])
        if cut < len(ids):
            st.stage_write(int(rows[b]), cut, ids[cut:])
    st.apply()
    computed = torch.zeros(R, dtype=torch.int32)
    for b, s in enumerate(plan.seqs):
        computed[int(rows[b])] = s.num_cached
    dm = pkv.prepare_metadata_device(rows.to(torch.int32).to(DEV), computed.to(DEV),
                                     torch.ones(B, dtype=torch.int32, device=DEV), table, 16, maxb, B)
    hm = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v)
          for k, v in pkv.prepare_metadata(plan.seqs, 16, maxb).items()}
    outs = []
    for tens, meta in ((tens_a, dm), (tens_b, hm)):
        pkv.store(tens.k_new(), tens.v_new(), tens.k_cache(), tens.v_cache(), meta["slot_mapping"][:B])
        outs.append(pkv.decode(tens.q[0], tens.k_cache(), tens.v_cache(), meta["block_tables"],
                               meta["context_lens"][:B], scale_of(plan.d)))
    torch.cuda.synchronize()
    assert torch.equal(tens_a.pool.view(torch.int16), tens_b.pool.view(torch.int16)), "caches"
    assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16)), "outputs"
    om = oracle_meta(plan)
    O.default().store(host.k_cache(), host.v_cache(), host.k_new(), host.v_new(), om["slot_mapping"])
    assert_close(outs[0], oracle_attention(plan, host, om), "decode on device metadata")
