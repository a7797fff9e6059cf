"""ctypes binding of libpkv_probe.so (include/pkv_probe.h): the benchmark's
measurement probes.  They measure what the device sustains with the attention
kernels' access patterns and instructions; no attention result comes from
them.  Loading fails loudly when the library has not been built."""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(HERE, "libpkv_probe.so")

EXPORTS = ("pkv_probe_paged_read", "pkv_probe_read", "pkv_probe_copy", "pkv_probe_mfma")

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(PROBE_LIB_PATH):
        raise ImportError(f"{PROBE_LIB_PATH} is missing: build it with "
                          "`python -m paged_kv_cache_110_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.pkv_probe_paged_read.argtypes = [P, P, P, I32, I32, I32, I32, I32, P, I32, I32, P]
    lib.pkv_probe_read.argtypes = [P, I64, P, I32, P]
    lib.pkv_probe_copy.argtypes = [P, P, I64, P]
    lib.pkv_probe_mfma.argtypes = [P, I32, I32, I32, I32, I32, P]
    for name in EXPORTS:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(name: str, rc: int) -> None:
    if rc != 0:
        raise RuntimeError(f"{name} failed with status {rc}")


def pages_of(block_tables: torch.Tensor, context_lens: torch.Tensor, block_size: int) -> torch.Tensor:
    """The (physical block, tokens used) pair of every page a decode over these
    tables reads, as a host int32 [num_pages, 2] tensor."""
    bt, cl = block_tables.cpu(), context_lens.cpu().tolist()
    out = []
    for b, n in enumerate(cl):
        for j in range(-(-n // block_size)):
            out.append((int(bt[b, j]), min(block_size, n - j * block_size)))
    return torch.tensor(out, dtype=torch.int32).reshape(-1, 2)


def paged_read(k_cache, v_cache, pages: torch.Tensor, sink: torch.Tensor,
               nontemporal: bool = True, group_heads: bool = False) -> None:
    nb, bs, H_kv, d = k_cache.shape
    _check("pkv_probe_paged_read", load().pkv_probe_paged_read(
        k_cache.data_ptr(), v_cache.data_ptr(), pages.data_ptr(), pages.shape[0], nb, H_kv, d, bs,
        sink.data_ptr(), int(nontemporal), int(group_heads), _stream()))


def read(src: torch.Tensor, sink: torch.Tensor, nontemporal: bool = False) -> None:
    _check("pkv_probe_read", load().pkv_probe_read(
        src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(), int(nontemporal),
        _stream()))


def copy(dst: torch.Tensor, src: torch.Tensor) -> None:
    assert dst.numel() * dst.element_size() == src.numel() * src.element_size()
    _check("pkv_probe_copy", load().pkv_probe_copy(
        dst.data_ptr(), src.data_ptr(), src.numel() * src.element_size(), _stream()))


def mfma(sink: torch.Tensor, num_cus: int, waves_per_simd: int, iters: int, chains: int,
         f16: bool = False) -> int:
    """Launch the MFMA loop; returns the flops it performs."""
    assert sink.numel() >= num_cus * 4 * waves_per_simd
    _check("pkv_probe_mfma", load().pkv_probe_mfma(sink.data_ptr(), num_cus, waves_per_simd, iters,
                                                   chains, int(f16), _stream()))
    return num_cus * 4 * waves_per_simd * iters * chains * 32768
