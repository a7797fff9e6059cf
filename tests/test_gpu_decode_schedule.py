"""Decode parity on batches large enough that the kernel's work schedule hands
out dynamic shares (more than 64 16-token tiles per resident wavefront):
long segments cut into many pieces, batches beyond the sequences whose
offsets the kernel keeps in LDS, padding rows, and a workspace reused across
calls.  Every output is compared with the float64 oracle."""
import pytest
import torch

import paged_kv_cache_110_amd as pkv
from gpu_harness import (assert_bits_equal, assert_close, cpu_copy, device_meta, gpu_store, log,
                         oracle_attention, oracle_meta, oracle_store, scale_of)
from workloads import custom_plan, make_tensors

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _plan(lens, bs, H_q, H_kv, d, seed):
    cap = -(-max(lens) // bs)
    return custom_plan([(n - 1, 1) for n in lens], bs, H_q, H_kv, d, seed=seed, extra_blocks=3,
                       max_blocks_per_seq=cap)


def _run(plan, pad_rows=(), seed=None, workspace=None, calls=1):
    tens = make_tensors(plan, DEV, poison=True, seed=seed)
    host = cpu_copy(tens)
    meta = pkv.prepare_metadata(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    ometa = oracle_meta(plan)
    for r in pad_rows:  # padding rows of a captured batch: slot -1, context 0
        meta["slot_mapping"][r] = -1
        meta["context_lens"][r] = 0
        ometa["slot_mapping"][r] = -1
        ometa["context_lens"][r] = 0
    dmeta = device_meta(meta, DEV)
    gpu_store(plan, tens, dmeta)
    outs = []
    for _ in range(calls):
        out = pkv.decode(tens.q[0], tens.k_cache(), tens.v_cache(), dmeta["block_tables"],
                         dmeta["context_lens"], scale_of(plan.d), workspace=workspace)
        outs.append(out.clone())
    torch.cuda.synchronize()
    oracle_store(host, ometa)
    ref = oracle_attention(plan, host, ometa)
    assert_bits_equal(tens.k_cache(), host.k_cache(), "k_cache after store")
    for r in pad_rows:
        assert torch.equal(outs[0][r].cpu(), torch.zeros_like(outs[0][r].cpu())), "padding row"
    return outs, ref


DYN_GEOMS = [  # (block_size, H_q, H_kv, d)
    (256, 16, 8, 128), (256, 32, 8, 128), (64, 8, 8, 128), (16, 64, 8, 128), (32, 16, 4, 64),
    (256, 8, 1, 64),
]


@pytest.mark.parametrize("geom", DYN_GEOMS, ids=lambda g: "bs%d_Hq%d_Hkv%d_d%d" % g)
def test_decode_dynamic_schedule(geom):
    bs, H_q, H_kv, d = geom
    g = torch.Generator().manual_seed(11 + sum(geom))
    # enough tiles that the schedule goes dynamic for every head count: a few
    # very long sequences (many pieces each), many mid-size ones, some short
    units_wanted = 160_000
    lens = [30_000, 17, 1, 9_000]
    while sum(-(-n // 16) for n in lens) * H_kv < units_wanted:
        lens.append(int(torch.randint(1, 6_000, (1,), generator=g)))
    log(f"dynamic schedule {geom}: B={len(lens)}, {sum(lens)} keys")
    plan = _plan(lens, bs, H_q, H_kv, d, seed=sum(geom))
    outs, ref = _run(plan, pad_rows=(5, 6))
    assert_close(outs[0], ref, f"decode dynamic {geom}")


def test_decode_beyond_cached_offsets():
    # more sequences than the kernel keeps offsets for in LDS (512): the share
    # search falls back to scanning context_lens
    g = torch.Generator().manual_seed(5)
    lens = [int(x) for x in torch.randint(1, 700, (1100,), generator=g)]
    lens[600] = 20_000  # a long one past the cached range
    log(f"decode with {len(lens)} sequences")
    plan = _plan(lens, 16, 16, 8, 128, seed=5)
    outs, ref = _run(plan, pad_rows=(3, 513, 1000))
    assert_close(outs[0], ref, "decode B=1100")


def test_decode_workspace_reuse_is_deterministic():
    # the share counter lives in the workspace: back-to-back calls on one
    # workspace must each see it reset and give bit-identical results
    g = torch.Generator().manual_seed(9)
    lens = [int(x) for x in torch.randint(100, 4000, (200,), generator=g)]
    plan = _plan(lens, 256, 16, 8, 128, seed=9)
    nbytes = pkv.decode_workspace_size(plan.B, plan.H_q, plan.H_kv, plan.d, plan.block_size,
                                       plan.max_blocks_per_seq)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device=DEV)
    log(f"workspace reuse: B={plan.B}, {nbytes} workspace bytes, 3 calls")
    outs, ref = _run(plan, workspace=ws, calls=3)
    for i in (1, 2):
        assert torch.equal(outs[0].view(torch.int16), outs[i].view(torch.int16)), f"call {i}"
    assert_close(outs[0], ref, "decode with a reused workspace")


@pytest.mark.parametrize("H_q", [16, 32], ids=["G2_valu", "G4_mfma"])
def test_decode_many_short_sequences(H_q):
    # four times as many sequences as resident wavefronts, most shorter than
    # one 16-token tile, with zero-length padding rows spread over the batch
    # (inside and beyond the sequences whose offsets sit in LDS)
    g = torch.Generator().manual_seed(21 + H_q)
    lens = [int(x) for x in torch.randint(1, 65, (8192,), generator=g)]
    log(f"decode with {len(lens)} short sequences, H_q {H_q}")
    plan = _plan(lens, 16, H_q, 8, 128, seed=21 + H_q)
    outs, ref = _run(plan, pad_rows=(0, 511, 512, 4095, 8191))
    assert_close(outs[0], ref, f"decode B=8192 H_q={H_q}")
