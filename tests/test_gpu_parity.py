"""HIP path (through the C ABI) against the CPU oracle, on the GPU.

Bars: the store and the cache contents bit-exact; each attention output
within 1e-2 of the float64 oracle or equal to one of the two bf16 values that
bracket the oracle's value (``gpu_harness.within_bar``).  Small cases and the
decode workloads at full size compare every output; the full-size prefill
workloads compare every row of the shared-prefix sequences plus sampled rows
of the rest, in the same launch configuration the benchmark times.
"""
import math

import pytest
import torch

import oracle as O
import paged_kv_cache_110_amd as pkv
from gpu_harness import (TOL, assert_bits_equal, assert_close, cpu_copy, device_meta,
                         gpu_attention, gpu_store, log, oracle_attention, oracle_meta,
                         oracle_store, scale_of)
from workloads import SeqState, custom_plan, make_plan, make_tensors

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _full_check(plan, seed=None, poison=True, tweak=None):
    """Store + attention on GPU and oracle; every output and the whole cache compared."""
    tens = make_tensors(plan, DEV, poison=poison, seed=seed)
    host = cpu_copy(tens)
    meta = pkv.prepare_metadata(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    ometa = oracle_meta(plan)
    if tweak:
        tweak(meta, ometa)
    dmeta = device_meta(meta, DEV)
    gpu_store(plan, tens, dmeta)
    out = gpu_attention(plan, tens, dmeta)
    torch.cuda.synchronize()
    oracle_store(host, ometa)
    ref = oracle_attention(plan, host, ometa)
    assert_bits_equal(tens.k_cache(), host.k_cache(), "k_cache after store")
    assert_bits_equal(tens.v_cache(), host.v_cache(), "v_cache after store")
    assert_close(out, ref, f"{plan.kind} B={plan.B} G={plan.H_q // plan.H_kv} d={plan.d} "
                           f"bs={plan.block_size}")
    return tens, out, ref


def test_tiny_decode_config():
    log("tiny_decode config: store + decode")
    plan = make_plan("tiny_decode")
    tens, out, ref = _full_check(plan)
    # context length 1: the output is the stored value row, exactly
    G = plan.H_q // plan.H_kv
    for h in range(plan.H_q):
        assert torch.equal(out[0, h].cpu().float(), tens.v_new()[0, h // G].cpu().float())


DECODE_GEOMS = [  # (block_size, H_q, H_kv, d)
    (16, 4, 2, 64), (16, 8, 1, 64), (32, 16, 4, 64), (16, 8, 8, 64),
    (256, 16, 8, 128), (16, 4, 4, 128), (64, 32, 8, 128), (256, 64, 8, 128),
    (1024, 16, 2, 128),
]


@pytest.mark.parametrize("geom", DECODE_GEOMS, ids=lambda g: "bs%d_Hq%d_Hkv%d_d%d" % g)
def test_decode_random_shapes(geom):
    bs, H_q, H_kv, d = geom
    log(f"decode geom {geom}")
    g = torch.Generator().manual_seed(sum(geom))
    lens = [1, 2, bs, bs + 1, 3 * bs - 1, 257, 1000, 3001]
    lens += [int(x) for x in torch.randint(1, 3500, (6,), generator=g)]
    plan = custom_plan([(n - 1, 1) for n in lens], bs, H_q, H_kv, d, seed=sum(geom),
                       extra_blocks=5, max_blocks_per_seq=-(-3600 // bs))

    def pad_rows(meta, ometa):
        # sequence 3 becomes a padding row of a captured batch: slot -1, context 0
        meta["slot_mapping"][3] = -1
        meta["context_lens"][3] = 0
        ometa["slot_mapping"][3] = -1
        ometa["context_lens"][3] = 0

    tens, out, ref = _full_check(plan, tweak=pad_rows)
    assert torch.equal(out[3].cpu(), torch.zeros_like(out[3].cpu())), "padding row must be zero"


PREFILL_GEOMS = [  # (block_size, H_q, H_kv, d)
    (16, 4, 2, 64), (16, 8, 8, 64), (256, 16, 8, 128), (32, 16, 2, 128),
    (16, 8, 1, 128), (256, 32, 4, 64), (1024, 8, 2, 128),
]


@pytest.mark.parametrize("geom", PREFILL_GEOMS, ids=lambda g: "bs%d_Hq%d_Hkv%d_d%d" % g)
def test_prefill_random_shapes(geom):
    bs, H_q, H_kv, d = geom
    log(f"prefill geom {geom}")
    specs = [(0, 1), (0, 37), (5, 64), (bs, 130), (3 * bs + 7, 300), (2 * bs, 2 * bs),
             (64, 0), (700, 1), (0, 513)]
    plan = custom_plan(specs, bs, H_q, H_kv, d, seed=7 + bs, extra_blocks=3, kind="prefill")
    _full_check(plan)



@pytest.mark.parametrize("geom", [(16, 16, 8, 128), (32, 64, 8, 64)],
                         ids=lambda g: "bs%d_Hq%d_Hkv%d_d%d" % g)
def test_prefill_many_tiny_sequences(geom):
    # thousands of sequences of 0-4 new tokens behind 0-300 cached ones: one
    # partly filled query tile each (or none), most keys behind a cached prefix
    bs, H_q, H_kv, d = geom
    g = torch.Generator().manual_seed(17 + bs)
    specs = [(int(c), int(n)) for c, n in zip(torch.randint(0, 301, (3000,), generator=g),
                                              torch.randint(0, 5, (3000,), generator=g))]
    log(f"prefill of {len(specs)} tiny sequences, geom {geom}")
    plan = custom_plan(specs, bs, H_q, H_kv, d, seed=17 + bs, extra_blocks=3, kind="prefill")
    _full_check(plan)


HEAD_COUNT_GEOMS = [  # (block_size, H_q, H_kv, d): multi-head (G = 1) with many heads, odd KV head counts
    (16, 32, 32, 128), (64, 12, 3, 64), (32, 40, 5, 128), (256, 6, 3, 128),
]


@pytest.mark.parametrize("geom", HEAD_COUNT_GEOMS, ids=lambda g: "bs%d_Hq%d_Hkv%d_d%d" % g)
@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_unusual_head_counts(geom, kind):
    bs, H_q, H_kv, d = geom
    log(f"{kind} with H_q {H_q}, H_kv {H_kv}, d {d}, block size {bs}")
    if kind == "decode":
        specs = [(n - 1, 1) for n in (1, 17, 300, 2500, 64, 999)]
    else:
        specs = [(0, 1), (0, 77), (bs + 3, 200), (5, 0), (700, 130)]
    plan = custom_plan(specs, bs, H_q, H_kv, d, seed=31 + H_kv, extra_blocks=2, kind=kind)
    _full_check(plan)

def test_prefill_long_sequence():
    # more new tokens than the benchmark's sequences (several query tiles past 2048),
    # behind a cached prefix that ends mid-block
    log("prefill of 3000 new tokens after 333 cached")
    plan = custom_plan([(333, 3000), (0, 5)], 64, 4, 2, 64, seed=13, extra_blocks=2,
                       kind="prefill")
    _full_check(plan)


@pytest.mark.parametrize("geom", [(256, 16, 8, 128), (64, 32, 4, 64)],
                         ids=lambda g: "bs%d_Hq%d_Hkv%d_d%d" % g)
def test_prefill_long_context(geom):
    """A long prompt behind a long cached prefix (8192 + 8192 keys: 128 query tiles, 256 key
    tiles for the last ones), beside a short one; sampled rows, each the oracle's decode of
    that row (prefill of one row equals decode, pinned on the CPU)."""
    bs, H_q, H_kv, d = geom
    log(f"long-context prefill {geom}")
    plan = custom_plan([(8192, 8192), (0, 300)], bs, H_q, H_kv, d, seed=29, extra_blocks=2,
                       kind="prefill")
    tens = make_tensors(plan, DEV, poison=True)
    host = cpu_copy(tens)
    meta = pkv.prepare_metadata(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    dm = device_meta(meta, DEV)
    gpu_store(plan, tens, dm)
    out = gpu_attention(plan, tens, dm)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    ometa = oracle_meta(plan)
    oracle_store(host, ometa)
    rows, tables, ctx = [], [], []
    g = torch.Generator().manual_seed(31)
    for b, s in enumerate(plan.seqs):
        start = ometa["cu_seqlens_q"][b]
        edges = {0, 1, 63, 64, 65, s.num_new - 1}
        pick = {i for i in edges if i < s.num_new}
        pick |= set(torch.randint(0, s.num_new, (24,), generator=g).tolist())
        for i in sorted(pick):
            rows.append(start + i)
            tables.append(ometa["block_tables"][b])
            ctx.append(s.num_cached + i + 1)
    ref = O.default().decode(host.q[0][rows], host.k_cache(), host.v_cache(), tables, ctx,
                             scale_of(d))
    assert_close(out[rows], ref, f"long-context prefill {geom}, {len(rows)} sampled rows")

def test_prefill_shared_prefix():
    log("prefill with shared prefix blocks")
    bs = 16
    specs = [(64, 40), (64, 40), (96, 3), (64, 1)]
    plan = custom_plan(specs, bs, 8, 2, 128, seed=3, share_first=(2, 4), kind="prefill")
    tens = make_tensors(plan, DEV, poison=True)
    tens.kv_new[0, 40:80] = tens.kv_new[0, 0:40]
    tens.q[0, 40:80] = tens.q[0, 0:40]
    host = cpu_copy(tens)
    meta = device_meta(pkv.prepare_metadata(plan.seqs, bs, plan.max_blocks_per_seq), DEV)
    gpu_store(plan, tens, meta)
    out = gpu_attention(plan, tens, meta)
    ometa = oracle_meta(plan)
    oracle_store(host, ometa)
    ref = oracle_attention(plan, host, ometa)
    assert_close(out, ref, "shared prefix prefill")
    assert torch.equal(out[0:40], out[40:80])


def _relabelled(plan, tens, perm):
    pool = torch.empty_like(tens.pool)
    pool[:, :, perm.to(pool.device)] = tens.pool
    seqs = [SeqState(tuple(int(perm[p]) for p in s.block_ids), s.num_cached, s.num_new)
            for s in plan.seqs]
    return pool, seqs


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_permutation_invariance_and_determinism(kind):
    log(f"physical-id relabelling, determinism, read-only caches: {kind}")
    bs = 16
    if kind == "decode":
        plan = custom_plan([(n - 1, 1) for n in (5, 40, 300, 1200)], bs, 8, 2, 128, seed=1,
                           extra_blocks=4)
    else:
        plan = custom_plan([(0, 50), (48, 70), (200, 9)], bs, 8, 2, 128, seed=2, extra_blocks=4,
                           kind="prefill")
    tens = make_tensors(plan, DEV, poison=True)
    dm = device_meta(pkv.prepare_metadata(plan.seqs, bs, plan.max_blocks_per_seq), DEV)
    gpu_store(plan, tens, dm)
    before = tens.pool.clone()
    out1 = gpu_attention(plan, tens, dm)
    out2 = gpu_attention(plan, tens, dm)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2), "two identical calls differ"
    assert torch.equal(before.view(torch.int16), tens.pool.view(torch.int16)), "attention wrote the cache"
    perm = torch.randperm(plan.num_blocks, generator=torch.Generator().manual_seed(5))
    pool2, seqs2 = _relabelled(plan, tens, perm)
    dm2 = device_meta(pkv.prepare_metadata(seqs2, bs, plan.max_blocks_per_seq), DEV)
    tens.pool = pool2
    out3 = gpu_attention(plan, tens, dm2)
    torch.cuda.synchronize()
    assert torch.equal(out1, out3), "relabelling physical blocks changed the GPU output"


# ------------------------------------------------------------ full sizes


@pytest.mark.parametrize("name", ["qwen3_decode", "long_decode", "wide_gqa_decode"])
def test_full_size_decode(name):
    """The whole workload, every output compared: the oracle's decode of all
    sequences takes well under a second on the host cores."""
    log(f"full-size {name}")
    plan = make_plan(name)
    tens = make_tensors(plan, DEV, poison=True)
    host = cpu_copy(tens)
    meta = pkv.prepare_metadata(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    dm = device_meta(meta, DEV)
    gpu_store(plan, tens, dm)
    out = gpu_attention(plan, tens, dm)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    ometa = oracle_meta(plan)
    oracle_store(host, ometa)
    assert_bits_equal(tens.k_cache(), host.k_cache(), f"{name} k_cache after store")
    assert_bits_equal(tens.v_cache(), host.v_cache(), f"{name} v_cache after store")
    ref = oracle_attention(plan, host, ometa)
    assert_close(out, ref, f"{name} all {plan.B} sequences")


def test_decode_one_very_long_sequence():
    """A 131072-token sequence beside a 37-token one: each KV head of the long
    sequence is cut into many pieces over the device's wavefronts, which the
    merge combines.  Every output, against the oracle."""
    log("decode of a 131072-token sequence beside a 37-token one")
    plan = custom_plan([(131071, 1), (36, 1)], 256, 16, 8, 128, seed=41, extra_blocks=2)
    _full_check(plan)


def test_full_size_prefix_prefill():
    log("full-size prefix_prefill")
    plan = make_plan("prefix_prefill")
    tens = make_tensors(plan, DEV, poison=True)
    host = cpu_copy(tens)
    meta = pkv.prepare_metadata(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    dm = device_meta(meta, DEV)
    gpu_store(plan, tens, dm)
    out = gpu_attention(plan, tens, dm)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    ometa = oracle_meta(plan)
    oracle_store(host, ometa)
    assert_bits_equal(tens.k_cache(), host.k_cache(), "prefix_prefill k_cache after store")
    assert_bits_equal(tens.v_cache(), host.v_cache(), "prefix_prefill v_cache after store")
    # sampled query rows: row i of sequence b is attention over keys 0..c+i, which the
    # oracle's decode computes one by one (prefill of one row == decode, pinned on CPU)
    rows, tables, ctx = [], [], []
    g = torch.Generator().manual_seed(4)
    for b in [0, 3, 4, 9, 15]:
        s = plan.seqs[b]
        start = ometa["cu_seqlens_q"][b]
        pick = {0, s.num_new - 1} | set(torch.randint(0, s.num_new, (40,), generator=g).tolist())
        for i in sorted(pick):
            rows.append(start + i)
            tables.append(ometa["block_tables"][b])
            ctx.append(s.num_cached + i + 1)
    ref = O.default().decode(host.q[0][rows], host.k_cache(), host.v_cache(), tables, ctx,
                             scale_of(plan.d))
    assert_close(out[rows], ref, "prefix_prefill sampled rows")
    # sequences 0..3 share their first 8 blocks: every row of the four, by the
    # oracle's own prefill over those sequences
    assert all(plan.seqs[b].block_ids[:8] == plan.seqs[0].block_ids[:8] for b in range(4))
    cq, ck = ometa["cu_seqlens_q"][:5], ometa["cu_seqlens_k"][:5]
    ref4 = O.default().prefill(host.q[0][: cq[4]], host.k_cache(), host.v_cache(),
                               ometa["block_tables"][:4], cq, ck, scale_of(plan.d))
    assert_close(out[: cq[4]], ref4, f"prefix_prefill all {cq[4]} rows of the shared-prefix sequences")


def test_full_size_full_step():
    """28 layers of store + decode on views of one [2, 28, blocks, 256, 8, 128] pool."""
    log("full-size full_step (28 layers)")
    plan = make_plan("full_step")
    tens = make_tensors(plan, DEV, poison=True)
    check_layers = [0, 13, 27]
    host = cpu_copy(tens, layers=check_layers)
    meta = pkv.prepare_metadata(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    dm = device_meta(meta, DEV)
    outs = []
    for layer in range(plan.layers):
        gpu_store(plan, tens, dm, layer)
        outs.append(gpu_attention(plan, tens, dm, layer))
    torch.cuda.synchronize()
    ometa = oracle_meta(plan)
    for j, layer in enumerate(check_layers):
        log(f"full_step layer {layer}")
        O.default().store(host.k_cache(j), host.v_cache(j), host.k_new(layer), host.v_new(layer),
                          ometa["slot_mapping"])
        assert_bits_equal(tens.k_cache(layer), host.k_cache(j), f"layer {layer} k_cache")
        assert_bits_equal(tens.v_cache(layer), host.v_cache(j), f"layer {layer} v_cache")
        ref = O.default().decode(host.q[layer], host.k_cache(j), host.v_cache(j),
                                 ometa["block_tables"], ometa["context_lens"], scale_of(plan.d))
        assert torch.isfinite(outs[layer].float()).all()
        assert_close(outs[layer], ref, f"full_step layer {layer}, all {plan.B} sequences")
    del tens
    torch.cuda.empty_cache()


PACKED_GEOMS = [  # (H_q, H_kv, d)
    (16, 8, 128), (8, 8, 64), (32, 8, 128), (8, 1, 128), (16, 4, 64),
]


@pytest.mark.parametrize("geom", PACKED_GEOMS, ids=lambda g: "Hq%d_Hkv%d_d%d" % g)
def test_prefill_packed(geom):
    """Varlen prefill over packed K/V rows (no block table), from views of one
    fused QKV buffer per token, with and without a cached prefix."""
    H_q, H_kv, d = geom
    log(f"packed prefill {geom}")
    g = torch.Generator().manual_seed(3 + H_q + d)
    specs = [(0, 1), (0, 64), (0, 65), (0, 700), (130, 70), (64, 1), (0, 2), (300, 513), (0, 0)]
    nq = [n for _, n in specs]
    nk = [c + n for c, n in specs]
    cu_q = [0]
    cu_k = [0]
    for a, b in zip(nq, nk):
        cu_q.append(cu_q[-1] + a)
        cu_k.append(cu_k[-1] + b)
    width = (H_q + 2 * H_kv) * d
    qbuf = torch.randn(cu_q[-1], width, generator=g).to(torch.bfloat16)
    kvbuf = torch.randn(cu_k[-1], width, generator=g).to(torch.bfloat16)
    q = qbuf[:, : H_q * d].view(-1, H_q, d)
    k = kvbuf[:, H_q * d: (H_q + H_kv) * d].view(-1, H_kv, d)
    v = kvbuf[:, (H_q + H_kv) * d:].view(-1, H_kv, d)
    dq, dk, dv = (t.to(DEV) for t in (qbuf, kvbuf, kvbuf))
    gq = dq[:, : H_q * d].view(-1, H_q, d)
    gk = dk[:, H_q * d: (H_q + H_kv) * d].view(-1, H_kv, d)
    gv = dv[:, (H_q + H_kv) * d:].view(-1, H_kv, d)
    cq = torch.tensor(cu_q, dtype=torch.int32, device=DEV)
    ck = torch.tensor(cu_k, dtype=torch.int32, device=DEV)
    out = pkv.prefill_varlen_packed(gq, gk, gv, cq, ck, max(nq), max(nk), scale_of(d))
    torch.cuda.synchronize()
    ref = O.default().prefill_packed(q, k, v, cu_q, cu_k, scale_of(d))
    assert_close(out, ref, f"packed prefill {geom}")


def test_full_size_packed_prefill():
    """The packed prefill workload at full size, launched as the benchmark times
    it (q/k/v as views of one fused buffer); sampled query rows are checked
    against the oracle's decode through a one-token-per-block table (row i of
    sequence b attends key rows cu[b] .. cu[b] + i)."""
    from workloads.packed import PACKED_PREFILL as cfg, make_packed, split_fused

    log("full-size packed_prefill")
    lens, cu, fused = make_packed(DEV)
    q, k, v = split_fused(fused)
    mx = max(lens)
    out = pkv.prefill_varlen_packed(q, k, v, cu, cu, mx, mx, scale_of(cfg["d"]))
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
    hq, hk, hv = (t.cpu() for t in (q, k, v))
    T, H_kv, d = hk.shape
    kc = hk.contiguous().view(T, 1, H_kv, d)
    vc = hv.contiguous().view(T, 1, H_kv, d)
    cu_h = cu.cpu().tolist()
    g = torch.Generator().manual_seed(6)
    rows, ctx, first = [], [], []
    for b in [0, 5, 11, 15, max(range(len(lens)), key=lambda i: lens[i])]:
        n = lens[b]
        pick = {0, n - 1} | set(torch.randint(0, n, (12,), generator=g).tolist())
        for i in sorted(pick):
            rows.append(cu_h[b] + i)
            ctx.append(i + 1)
            first.append(cu_h[b])
    width = max(ctx)
    tables = [[f + j if j < c else -1 for j in range(width)] for f, c in zip(first, ctx)]
    ref = O.default().decode(hq[rows].contiguous(), kc, vc, tables, ctx, scale_of(d))
    assert_close(out[rows], ref, "packed_prefill sampled rows")


def _scale_rows(t, rows, factor):
    """Multiply bf16 rows in place (result rounded to bf16)."""
    t[rows] = (t[rows].float() * factor).to(torch.bfloat16)


def test_prefill_v_beyond_fp16_range():
    """V anywhere in bf16's range: sequence 0's V is scaled by 2^15 (values up
    to about 1.3e5, beyond fp16's largest, 65504), sequence 1's by 2^-20
    (below 2^-14: fp16 subnormals), sequence 2 keeps N(0, 1).  Paged and
    packed.  Attention is linear in V, so a sequence whose V is scaled by F is
    held to the bar at its own scale: out / F against the oracle's / F (F a
    power of two: the division is exact and keeps bf16 values bf16)."""
    log("prefill with V beyond fp16's range and below its normal range")
    bs = 16
    specs = [(40, 70), (17, 33), (64, 50)]
    plan = custom_plan(specs, bs, 8, 2, 128, seed=21, extra_blocks=2, kind="prefill")
    tens = make_tensors(plan, DEV, poison=True)
    D = plan.H_kv * plan.d
    factors = [2.0 ** 15, 2.0 ** -20, 1.0]
    meta = pkv.prepare_metadata(plan.seqs, bs, plan.max_blocks_per_seq)
    row0 = 0
    for s, f in zip(plan.seqs, factors):
        blocks = torch.tensor(s.block_ids, dtype=torch.long, device=DEV)
        vc = tens.pool[1, 0]
        vc[blocks] = (vc[blocks].float() * f).to(torch.bfloat16)
        _scale_rows(tens.kv_new[0, :, D:], slice(row0, row0 + s.num_new), f)
        row0 += s.num_new
    vmax = tens.pool[1, 0].float().nan_to_num(0).abs().max().item()
    assert vmax > 65504, vmax  # some V values really are beyond fp16's range
    host = cpu_copy(tens)
    dm = device_meta(meta, DEV)
    gpu_store(plan, tens, dm)
    out = gpu_attention(plan, tens, dm)
    torch.cuda.synchronize()
    ometa = oracle_meta(plan)
    oracle_store(host, ometa)
    ref = oracle_attention(plan, host, ometa)
    cq = ometa["cu_seqlens_q"]

    def check(o, r, what):
        for b, f in enumerate(factors):
            rows = slice(cq[b], cq[b + 1])
            got = o[rows].detach().float().cpu().double()
            assert_close(got / f, r[rows] / f, f"{what}, V scaled by 2^{round(math.log2(f))} "
                                               f"(sequence {b}), judged at that scale")

    check(out, ref, "paged prefill")

    # the packed form over the same rows: keys of each sequence gathered in order
    ks, vs, cu_k = [], [], [0]
    for s in plan.seqs:
        rows = torch.tensor([s.block_ids[j // bs] * bs + j % bs for j in range(s.total)],
                            dtype=torch.long)
        ks.append(host.k_cache().reshape(-1, plan.H_kv, plan.d)[rows])
        vs.append(host.v_cache().reshape(-1, plan.H_kv, plan.d)[rows])
        cu_k.append(cu_k[-1] + s.total)
    k, v = torch.cat(ks), torch.cat(vs)
    cq_t = torch.tensor(cq, dtype=torch.int32, device=DEV)
    ck_t = torch.tensor(cu_k, dtype=torch.int32, device=DEV)
    outp = pkv.prefill_varlen_packed(tens.q[0], k.to(DEV), v.to(DEV), cq_t, ck_t,
                                     max(s.num_new for s in plan.seqs),
                                     max(s.total for s in plan.seqs), scale_of(plan.d))
    torch.cuda.synchronize()
    refp = O.default().prefill_packed(host.q[0], k, v, cq, cu_k, scale_of(plan.d))
    check(outp, refp, "packed prefill")
