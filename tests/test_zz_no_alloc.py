"""pkv_sample_gumbel_noalloc (the entry point that allocates nothing: its
chunk keys go to a fixed per-device scratch array inside the library) against
pkv_sample_gumbel with a caller workspace, through the raw C ABI: the same
tokens, bit for bit, on two calls in a row, the second smaller than the first
(so it runs over what the first left in the scratch).  Sizes beyond the
scratch are refused on the host (tests/test_lib_abi.py, no GPU needed)."""
import ctypes

import pytest
import torch

from gpu_harness import log
from paged_kv_cache_110_amd import _lib
from workloads.sampling import make_logits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _inputs(B, V, bf16, pad, seed):
    g = torch.Generator().manual_seed(seed)
    rows = torch.randn(B, V + pad, generator=g) * 3.0
    logits = (rows.to(torch.bfloat16) if bf16 else rows).to(DEV)
    temps = (0.2 + 1.3 * torch.rand(B, generator=g)).to(DEV)
    temps[0] = 0.0  # a greedy row
    seeds = torch.randint(0, 2 ** 62, (B,), generator=g, dtype=torch.int64).to(DEV)
    offsets = torch.randint(0, 4096, (B,), generator=g, dtype=torch.int64).to(DEV)
    return logits[:, :V], temps, seeds, offsets


def _both(logits, temps, seeds, offsets):
    lib = _lib.load()
    B, V = logits.shape
    bf16 = int(logits.dtype == torch.bfloat16)
    stride = logits.stride(0)
    ref = torch.full((B,), -1, dtype=torch.int64, device=DEV)
    got = torch.full((B,), -2, dtype=torch.int64, device=DEV)
    ws_bytes = lib.pkv_sample_workspace_size(B, V)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    rc = lib.pkv_sample_gumbel(ref.data_ptr(), logits.data_ptr(), bf16, stride, B, V,
                               temps.data_ptr(), seeds.data_ptr(), offsets.data_ptr(),
                               ws.data_ptr(), ws_bytes, _stream())
    assert rc == 0, rc
    rc = lib.pkv_sample_gumbel_noalloc(got.data_ptr(), logits.data_ptr(), bf16, stride, B, V,
                                       temps.data_ptr(), seeds.data_ptr(), offsets.data_ptr(),
                                       _stream())
    assert rc == 0, rc
    torch.cuda.synchronize()
    return ref.cpu(), got.cpu()


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    log("no-alloc sampling: call 1, 256 x 151936 bf16 (the decode step's logits)")
    logits, temps, seeds, offsets = make_logits(DEV)
    ref, got = _both(logits, temps, seeds, offsets)
    assert (ref >= 0).all() and (ref < logits.shape[1]).all()
    assert torch.equal(ref, got), f"{int((ref != got).sum())} rows differ"
    log("no-alloc sampling: call 2, 37 x 50000 fp32 with padded rows (smaller)")
    logits, temps, seeds, offsets = _inputs(37, 50000, False, 12, 7)
    ref, got = _both(logits, temps, seeds, offsets)
    assert (ref >= 0).all() and (ref < 50000).all()
    assert torch.equal(ref, got), f"{int((ref != got).sum())} rows differ"
    assert got[0].item() == int(torch.argmax(logits[0].float()).item())  # T = 0: argmax
