"""The C-ABI library loads and exports what include/pkv.h declares; host-side
argument checks and the host metadata routine (CPU only, no kernel launches)."""
import ctypes
import os
import re

import pytest
import torch

import oracle as O
import paged_kv_cache_110_amd as pkv
from paged_kv_cache_110_amd import _lib
from workloads import SeqState, custom_plan, make_plan, CONFIG_ORDER

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert _declared() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    for name in _declared():
        assert hasattr(lib, name), name
    assert pkv.version() == 100


def test_status_strings():
    lib = _lib.load()
    for code in range(5):
        assert lib.pkv_status_string(code).decode().startswith("PKV_")
    assert b"unknown" in lib.pkv_status_string(99)


def _null_stream():
    return ctypes.c_void_p(0)


def test_store_argument_checks_before_launch():
    lib = _lib.load()
    buf = ctypes.create_string_buffer(4096 + 16)
    base = (ctypes.addressof(buf) + 15) // 16 * 16
    # num_tokens == 0: nothing to do
    assert lib.pkv_store(None, 0, None, 0, None, None, None, 0, 4, 16, 2, 64, None) == 0
    # null pointers
    assert lib.pkv_store(None, 128, None, 128, None, None, None, 1, 4, 16, 2, 64, None) == 1
    # block size not a power of two
    assert lib.pkv_store(base, 128, base, 128, base, base, base, 1, 4, 24, 2, 64, None) == 1
    # stride below the row size
    assert lib.pkv_store(base, 64, base, 128, base, base, base, 1, 4, 16, 2, 64, None) == 1
    # misaligned pointer
    assert lib.pkv_store(base + 2, 128, base, 128, base, base, base, 1, 4, 16, 2, 64, None) == 1


def test_store_decode_argument_checks_before_launch():
    """pkv_store_decode rejects what pkv_decode rejects, plus bad new-token rows,
    before any launch (so this runs without a GPU)."""
    lib = _lib.load()
    buf = ctypes.create_string_buffer(4096 + 16)
    p = (ctypes.addressof(buf) + 15) // 16 * 16
    row = 2 * 64  # H_kv * d

    def sd(key=None, kst=row, value=None, vst=row, B=2, H_q=4, H_kv=2, d=64, bs=16, ws=1 << 20,
           scale=0.125, wsp=None):
        key = p if key is None else key
        value = p if value is None else value
        return lib.pkv_store_decode(p, p, key, kst, value, vst, p, p, p, p, B, H_q, H_kv, d, 8, bs,
                                    3, scale, p if wsp is None else wsp, ws, None)

    assert lib.pkv_store_decode(p, p, None, row, p, row, p, p, p, p, 2, 4, 2, 64, 8, 16, 3,
                                0.125, p, 1 << 20, None) == 1   # null key
    assert lib.pkv_store_decode(p, p, p, row, None, row, p, p, p, p, 2, 4, 2, 64, 8, 16, 3,
                                0.125, p, 1 << 20, None) == 1   # null value
    assert sd(kst=row - 8) == 1           # key stride below H_kv * d
    assert sd(vst=row + 4) == 1           # value stride not a multiple of 8
    assert sd(key=p + 2) == 1             # misaligned key
    assert sd(value=p + 8) == 1           # misaligned value
    assert sd(B=0) == 1
    assert sd(H_q=6, H_kv=4) == 1         # H_q % H_kv != 0
    assert sd(bs=24) == 1                 # not a power of two
    assert sd(d=96) == 2                  # unsupported head size
    assert sd(scale=float("nan")) == 1
    ws = lib.pkv_decode_workspace_size(2, 4, 2, 64, 16, 3)
    assert ws > 0 and sd(ws=ws - 1) == 1  # the decode's workspace size applies

def test_attention_argument_checks_before_launch():
    lib = _lib.load()
    buf = ctypes.create_string_buffer(4096 + 16)
    p = (ctypes.addressof(buf) + 15) // 16 * 16
    args = dict(B=2, H_q=4, H_kv=2, d=64, nb=8, bs=16, maxb=3)

    def dec(**kw):
        a = {**args, **kw}
        return lib.pkv_decode(p, p, p, p, p, p, a["B"], a["H_q"], a["H_kv"], a["d"], a["nb"],
                              a["bs"], a["maxb"], 0.125, p, 1 << 20, None)

    assert dec(H_q=6, H_kv=4) == 1        # H_q % H_kv != 0
    assert dec(bs=48) == 1                # not a power of two
    assert dec(bs=8) == 1                 # below 16
    assert dec(B=0) == 1
    assert dec(d=96) == 2                 # unsupported head size
    assert dec(H_q=48, H_kv=3) == 2       # group of 16
    # too small a workspace
    ws = lib.pkv_decode_workspace_size(2, 4, 2, 64, 16, 1024)
    assert ws > 0
    assert lib.pkv_decode(p, p, p, p, p, p, 2, 4, 2, 64, 8, 16, 1024, 0.125, p, ws - 1, None) == 1
    assert lib.pkv_decode(p, p, p, p, p, p, 2, 4, 2, 64, 8, 16, 1024, 0.125, None, ws, None) == 1

    def pf(**kw):
        a = {**args, **kw}
        return lib.pkv_prefill_varlen(p, p, p, p, p, p, p, a["B"], 10, 10, 10, a["H_q"], a["H_kv"],
                                      a["d"], a["nb"], a["bs"], a["maxb"], 0.125, None)

    assert pf(H_q=6, H_kv=4) == 1
    assert pf(d=256) == 2
    nan, inf = float("nan"), float("inf")
    for bad in (0.0, -0.125, nan, inf):   # the prefill scale must be finite and positive
        assert lib.pkv_prefill_varlen(p, p, p, p, p, p, p, 2, 10, 10, 10, 4, 2, 64, 8, 16, 3,
                                      bad, None) == 1
    for bad in (nan, inf, -inf):          # the decode scale must be finite
        assert lib.pkv_decode(p, p, p, p, p, p, 2, 4, 2, 64, 8, 16, 3, bad, p, 1 << 20, None) == 1
    hk = (1 << 17) + 1                    # H_kv * d just above 2^24 elements per row
    assert pf(H_q=hk, H_kv=hk, d=128) == 2
    # more query tiles (of 128 / G positions) than the grid's 65535
    too_many = 65535 * 64 + 1
    assert lib.pkv_prefill_varlen(p, p, p, p, p, p, p, 2, 10, too_many, 10, 4, 2, 64, 8, 16, 3,
                                  0.125, None) == 2
    assert lib.pkv_prefill_varlen(p, p, p, p, p, p, p, 0, 0, 0, 0, 4, 2, 64, 8, 16, 3, 0.125,
                                  None) == 0  # nothing to do


def test_packed_prefill_argument_checks_before_launch():
    lib = _lib.load()
    buf = ctypes.create_string_buffer(4096 + 16)
    p = (ctypes.addressof(buf) + 15) // 16 * 16

    def pk(qs=512, ks=256, vs=256, B=2, tq=10, tk=10, mq=10, H_q=8, H_kv=4, d=64, q=p,
           scale=0.125):
        return lib.pkv_prefill_varlen_packed(p, q, qs, p, ks, p, vs, p, p, B, tq, tk, mq, mq,
                                             H_q, H_kv, d, scale, None)

    assert pk(B=0) == 0 and pk(tq=0) == 0 and pk(mq=0) == 0   # nothing to do
    assert pk(qs=256) == 1        # q stride below H_q * d
    assert pk(ks=250) == 1        # not a multiple of 8, below the row
    assert pk(vs=260) == 1        # not a multiple of 8
    assert pk(H_q=6) == 1         # H_q % H_kv
    assert pk(q=p + 2) == 1       # misaligned
    assert pk(tk=0) == 1          # no keys
    assert pk(B=-1) == 1
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert pk(scale=bad) == 1
    assert pk(d=96, qs=768, ks=384, vs=384) == 2
    assert pk(H_q=64, H_kv=4, qs=4096) == 2  # group of 16
    assert pk(mq=65535 * 128 // 2 + 1) == 2  # more than 65535 query tiles (G = 2)
    big = (1 << 24) + 8
    assert pk(ks=big) == 2 and pk(vs=big) == 2   # row strides past the 32-bit tile offsets


def test_workspace_size_formula():
    lib = _lib.load()
    # partial slots per share of the schedule, plus 16 bytes per (sequence, KV head)
    # (256-byte aligned) and the share counter's line
    a = lib.pkv_decode_workspace_size(16, 4, 2, 64, 16, 3)
    b = lib.pkv_decode_workspace_size(32, 4, 2, 64, 16, 3)
    assert a > 0 and b - a == 16 * 2 * 16
    c = lib.pkv_decode_workspace_size(16, 8, 2, 64, 16, 3)  # G = 4: twice the partial rows
    assert c > a
    # the schedule counts units in int32: tables too wide for that are refused
    assert lib.pkv_decode_workspace_size(4096, 16, 8, 128, 256, 1 << 16) == 0
    assert lib.pkv_decode_workspace_size(4, 4, 2, 96, 16, 3) == 0  # unsupported d
    assert lib.pkv_decode_workspace_size(4, 6, 4, 64, 16, 3) == 0  # H_q % H_kv


def _meta_equal(a, b):
    for k in ("slot_mapping", "context_lens", "cu_seqlens_q", "cu_seqlens_k"):
        if k in b:
            assert a[k].tolist() == list(b[k]), k
    assert a["block_tables"].tolist() == b["block_tables"]


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_prepare_metadata_matches_oracle(name):
    plan = make_plan(name)
    got = pkv.prepare_metadata(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    ref = O.prepare_prefill(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
    _meta_equal(got, ref)
    assert got["max_seqlen_q"] == ref["max_seqlen_q"]
    assert got["max_seqlen_k"] == ref["max_seqlen_k"]
    if plan.kind == "decode":
        _meta_equal(got, O.prepare_decode(plan.seqs, plan.block_size, plan.max_blocks_per_seq))


def test_prepare_metadata_edge_cases():
    # sequence with no new tokens, one with an unfilled block, empty batch
    seqs = [SeqState((3, 1), 20, 0), SeqState((0,), 0, 5), SeqState((2, 4, 5), 33, 2)]
    got = pkv.prepare_metadata(seqs, 16, 4)
    ref = O.prepare_prefill(seqs, 16, 4)
    _meta_equal(got, ref)
    empty = pkv.prepare_metadata([], 16, 4)
    assert empty["cu_seqlens_q"].tolist() == [0] and empty["max_seqlen_k"] == 0
    with pytest.raises(pkv.PkvError):  # too few blocks for 40 tokens
        pkv.prepare_metadata([SeqState((1, 2), 30, 10)], 16, 4)
    with pytest.raises(pkv.PkvError):  # more blocks than the table width
        pkv.prepare_metadata([SeqState((1, 2, 3), 30, 10)], 16, 2)
    with pytest.raises(pkv.PkvError):  # negative block id
        pkv.prepare_metadata([SeqState((1, -3), 20, 1)], 16, 2)
    with pytest.raises(pkv.PkvError):  # block size not a power of two >= 16
        pkv.prepare_metadata([SeqState((1,), 2, 1)], 24, 2)


def test_prepare_metadata_random_plans():
    g = torch.Generator().manual_seed(0)
    for trial in range(20):
        bs = [16, 32, 64, 256][trial % 4]
        B = int(torch.randint(1, 9, (1,), generator=g))
        specs = [(int(torch.randint(0, 700, (1,), generator=g)),
                  int(torch.randint(0, 300, (1,), generator=g))) for _ in range(B)]
        plan = custom_plan(specs, bs, 4, 2, 64, seed=trial, extra_blocks=trial % 3,
                           kind="prefill")
        got = pkv.prepare_metadata(plan.seqs, bs, plan.max_blocks_per_seq + trial % 2)
        ref = O.prepare_prefill(plan.seqs, bs, plan.max_blocks_per_seq + trial % 2)
        _meta_equal(got, ref)


# ------------------------------------------------------------ decode-graph step


def test_graph_bucket_matches_oracle():
    lib = _lib.load()
    for mb in (1, 2, 3, 7, 8, 9, 16, 17, 40, 100, 511, 512, 0, 513, -4):
        for batch in list(range(-1, min(mb, 70) + 3)) + [mb - 1, mb, mb + 1, 1000]:
            assert lib.pkv_decode_graph_bucket(mb, batch) == O.graph.bucket_for(mb, batch), (mb, batch)


def test_step_struct_layout_matches_c(tmp_path):
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = str(tmp_path / "step_layout")
    subprocess.run([gcc, "-std=c11", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(rocm, "include"),
                    os.path.join(ROOT, "tests", "native", "step_layout.c"), "-o", exe], check=True)
    lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    got = dict(line.split() for line in lines if line.strip())
    assert int(got.pop("size")) == ctypes.sizeof(_lib.DecodeStep)
    for name, off in got.items():
        assert getattr(_lib.DecodeStep, name).offset == int(off), name
    assert len(got) == len(_lib.DecodeStep._fields_)


def test_graph_argument_checks_before_any_hip_call():
    lib = _lib.load()
    handle = ctypes.c_void_p(0)
    assert lib.pkv_decode_graph_create(None, ctypes.byref(handle)) == 1
    step = _lib.DecodeStep()
    assert lib.pkv_decode_graph_create(ctypes.byref(step), None) == 1
    assert lib.pkv_decode_graph_create(ctypes.byref(step), ctypes.byref(handle)) == 1  # layers 0
    step.layers, step.max_batch = 1, 513  # above the graph limit
    assert lib.pkv_decode_graph_create(ctypes.byref(step), ctypes.byref(handle)) == 1
    step.max_batch = 8  # null buffers
    assert lib.pkv_decode_graph_create(ctypes.byref(step), ctypes.byref(handle)) == 1
    assert handle.value is None
    assert lib.pkv_decode_graph_replay(None, 1, None) == 1
    assert lib.pkv_decode_step_run(None, 1, None) == 1
    assert lib.pkv_decode_step_run(ctypes.byref(step), 1, None) == 1
    lib.pkv_decode_graph_destroy(None)  # no-op


# ------------------------------------------------- staged writes, device metadata


def test_pack_row_writes_round_trip():
    g = torch.Generator().manual_seed(4)
    R, C = 50, 64
    writes, used = [], set()
    while len(writes) < 40:
        r = int(torch.randint(0, R, (1,), generator=g))
        s0 = int(torch.randint(0, C, (1,), generator=g))
        n = int(torch.randint(0, C - s0 + 1, (1,), generator=g))
        cells = {(r, s0 + i) for i in range(n)}
        if cells & used:
            continue
        used |= cells
        writes.append((r, s0, [int(x) for x in torch.randint(-100, 10**6, (n,), generator=g)]))
    packed = pkv.pack_row_writes(writes, R, C).tolist()
    n, total = len(writes), sum(len(w[2]) for w in writes)
    assert len(packed) == 3 * n + 1 + total
    rows, starts, off = packed[:n], packed[n:2 * n], packed[2 * n:3 * n + 1]
    vals = packed[3 * n + 1:]
    assert off[0] == 0 and off[-1] == total
    back = [(rows[w], starts[w], vals[off[w]:off[w + 1]]) for w in range(n)]
    assert back == writes
    base = [[-7] * C for _ in range(R)]
    assert O.apply_row_writes([r[:] for r in base], back) == O.apply_row_writes([r[:] for r in base], writes)


def test_pack_row_writes_rejects_bad_writes():
    def rejects(writes, R=8, C=10):
        with pytest.raises(pkv.PkvError):
            pkv.pack_row_writes(writes, R, C)

    rejects([(1, 2, [1, 2, 3]), (1, 4, [9])])       # overlap in one row
    rejects([(8, 0, [1])])                          # row out of range
    rejects([(0, 8, [1, 2, 3])])                    # past the last column
    rejects([(-1, 0, [1])])
    pkv.pack_row_writes([(1, 2, [1, 2]), (1, 4, [9]), (2, 2, [5]), (3, 0, [])], 8, 10)  # adjacent: ok
    lib = _lib.load()
    size = ctypes.c_int64(0)
    rows = (ctypes.c_int32 * 1)(0)
    starts = (ctypes.c_int32 * 1)(0)
    lens = (ctypes.c_int32 * 1)(-1)
    assert lib.pkv_pack_row_writes(1, rows, starts, lens, None, 4, 4, None, 0, ctypes.byref(size)) == 1
    lens[0] = 2
    vals = (ctypes.c_int32 * 2)(5, 6)
    out = (ctypes.c_int32 * 5)()
    assert lib.pkv_pack_row_writes(1, rows, starts, lens, vals, 4, 4, out, 5, ctypes.byref(size)) == 1
    assert size.value == 6  # the size is reported even when the capacity is short
    out6 = (ctypes.c_int32 * 6)()
    assert lib.pkv_pack_row_writes(1, rows, starts, lens, vals, 4, 4, out6, 6, ctypes.byref(size)) == 0
    assert list(out6) == [0, 0, 0, 2, 5, 6]


def test_device_metadata_argument_checks_before_any_hip_call():
    lib = _lib.load()
    buf = ctypes.create_string_buffer(256)
    a = ctypes.addressof(buf)
    call = lib.pkv_prepare_metadata_device
    # B < 0, bad block size, table narrower than max_blocks_per_seq, no outputs
    assert call(-1, None, a, a, a, 4, 8, 16, 8, 0, a, a, a, None, a, None, None, None) == 1
    assert call(2, None, a, a, a, 4, 8, 24, 8, 0, a, a, a, None, a, None, None, None) == 1
    assert call(2, None, a, a, a, 4, 4, 16, 8, 0, a, a, a, None, a, None, None, None) == 1
    assert call(2, None, a, a, a, 4, 8, 16, 8, 0, None, a, a, None, a, None, None, None) == 1
    assert call(2, None, None, a, a, 4, 8, 16, 8, 4, a, a, a, None, a, None, None, None) == 1
    assert call(4097, None, a, a, a, 4, 8, 16, 8, 4, a, a, a, None, a, None, None, None) == 2
    assert lib.pkv_apply_row_writes(None, 4, 2, 4, None, 0, 0, None) == 0  # nothing to do
    assert lib.pkv_apply_row_writes(None, 4, 2, 4, None, 1, 3, None) == 1
    assert lib.pkv_apply_row_writes(a, 3, 2, 4, a, 1, 3, None) == 1  # stride below the width


def test_sample_argument_checks_before_any_hip_call():
    lib = _lib.load()
    buf = ctypes.create_string_buffer(4096 + 16)
    a = (ctypes.addressof(buf) + 15) // 16 * 16
    call = lib.pkv_sample_gumbel
    assert call(None, None, 1, 104, 0, 100, None, None, None, None, 0, None) == 0  # B == 0
    assert call(a, a, 1, 8, 2, 0, None, a, None, a, 4096, None) == 1             # V < 1
    assert call(a, a, 1, 96, 2, 100, None, a, None, a, 4096, None) == 1          # stride < V
    assert call(a, a, 1, 100, 2, 100, None, a, None, a, 4096, None) == 1         # bf16 stride % 8
    assert call(a, a, 0, 102, 2, 100, None, a, None, a, 4096, None) == 1         # fp32 stride % 4
    assert call(a, a + 2, 1, 104, 2, 100, None, a, None, a, 4096, None) == 1     # misaligned
    assert call(a, a, 1, 104, 2, 100, None, None, None, a, 4096, None) == 1      # no seeds
    assert call(a, a, 1, 104, 2, 100, None, a, None, a, 8, None) == 1            # short workspace
    assert call(a, a, 1, 104, 2, 100, None, a, None, a + 4, 4096, None) == 1     # workspace % 8
    assert lib.pkv_sample_workspace_size(2, 100) == 16
    assert lib.pkv_sample_workspace_size(3, 151936) == 3 * 38 * 8
    assert lib.pkv_sample_workspace_size(0, 10) == 0


def test_probe_library_exports_and_argument_checks():
    """libpkv_probe.so (the benchmark's ceiling probes) loads, exports what
    include/pkv_probe.h declares, and rejects bad arguments before any HIP call."""
    from paged_kv_cache_110_amd import probe

    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "pkv_probe.h")).read(),
                  flags=re.S)
    declared = sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))
    assert declared == sorted(probe.EXPORTS)
    lib = probe.load()
    for name in declared:
        assert hasattr(lib, name), name
    buf = ctypes.create_string_buffer(4096 + 16)
    p = (ctypes.addressof(buf) + 15) // 16 * 16
    # paged read: d, block size, null pointers, empty page list, misaligned cache
    assert lib.pkv_probe_paged_read(p, p, p, 1, 4, 8, 96, 256, p, 1, 0, None) == 1
    assert lib.pkv_probe_paged_read(p, p, p, 1, 4, 8, 128, 48, p, 0, 1, None) == 1
    assert lib.pkv_probe_paged_read(None, p, p, 1, 4, 8, 128, 256, p, 1, 0, None) == 1
    assert lib.pkv_probe_paged_read(p, p, p, 0, 4, 8, 128, 256, p, 1, 0, None) == 1
    assert lib.pkv_probe_paged_read(p + 2, p, p, 1, 4, 8, 128, 256, p, 1, 0, None) == 1
    assert lib.pkv_probe_paged_read(p, p, p, 1, 4, 32, 128, 256, p, 1, 1, None) == 1  # grouped, H_kv > 16
    # read / copy: sizes that are not whole 16-byte chunks, misaligned buffers
    assert lib.pkv_probe_read(p, 24, p, 1, None) == 1
    assert lib.pkv_probe_read(p + 8, 32, p, 0, None) == 1
    assert lib.pkv_probe_copy(p, p, 0, None) == 1
    assert lib.pkv_probe_copy(p + 4, p, 32, None) == 1
    # mfma: chain counts and occupancies outside the supported set
    assert lib.pkv_probe_mfma(p, 256, 2, 10, 3, 0, None) == 1
    assert lib.pkv_probe_mfma(p, 256, 9, 10, 4, 0, None) == 1
    assert lib.pkv_probe_mfma(None, 256, 2, 10, 4, 0, None) == 1


def test_probe_page_list():
    """The probe's page list holds one (physical block, tokens used) pair per
    page a decode reads: whole pages, then the remainder of the last."""
    from paged_kv_cache_110_amd.probe import pages_of

    bt = torch.tensor([[5, 2, -1], [7, -1, -1], [1, 3, 4]], dtype=torch.int32)
    cl = torch.tensor([17, 16, 33], dtype=torch.int32)
    assert pages_of(bt, cl, 16).tolist() == [[5, 16], [2, 1], [7, 16], [1, 16], [3, 16], [4, 1]]


def test_sample_noalloc_refuses_sizes_beyond_its_scratch():
    """pkv_sample_gumbel_noalloc: the fixed scratch holds 2^17 chunk keys;
    larger calls return PKV_ESCRATCH on the host, before any HIP call."""
    lib = _lib.load()
    buf = ctypes.create_string_buffer(4096 + 16)
    p = (ctypes.addressof(buf) + 15) // 16 * 16
    V = 151936
    # bf16 chunks are 8192 logits (19 per row), fp32 chunks 4096 (38 per row)
    assert lib.pkv_sample_gumbel_noalloc(p, p, 1, V, 6899, V, None, p, None, None) == _lib.PKV_ESCRATCH
    assert lib.pkv_sample_gumbel_noalloc(p, p, 0, V, 3450, V, None, p, None, None) == _lib.PKV_ESCRATCH
    assert lib.pkv_sample_gumbel_noalloc(p, p, 1, V, 65536, V, None, p, None, None) == _lib.PKV_EINVAL
    assert lib.pkv_sample_gumbel_noalloc(p, p, 1, V, 0, V, None, p, None, None) == 0  # nothing to do
    assert lib.pkv_sample_gumbel_noalloc(None, p, 1, V, 4, V, None, p, None, None) == _lib.PKV_EINVAL
    assert lib.pkv_sample_gumbel_noalloc(p, p + 2, 1, V, 4, V, None, p, None, None) == _lib.PKV_EINVAL
    assert lib.pkv_sample_gumbel_noalloc(p, p, 1, V - 1, 4, V, None, p, None, None) == _lib.PKV_EINVAL
