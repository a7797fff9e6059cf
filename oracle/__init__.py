"""CPU oracle for paged-KV store and attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never loads it and shares no code
with it: the C part (``pkv_oracle.c``) is compiled by gcc into its own shared
object, the metadata loops live in ``metadata.py`` and the decode-graph bucket
rule in ``graph.py``.

Inputs are CPU torch tensors (bf16 data is passed as its raw 16-bit patterns);
attention outputs come back as float64 tensors.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np
import torch

from . import graph
from .metadata import apply_row_writes, prepare_decode, prepare_from_state, prepare_prefill

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "pkv_oracle.c")

ERRORS = {
    0: "ok",
    1: "inconsistent shape arguments",
    2: "slot outside [-1, num_blocks*block_size)",
    3: "duplicate slot",
    4: "block table entry outside [0, num_blocks) for a key that is read",
    5: "length negative or beyond the block table",
    6: "out of memory",
}


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle error {code}: {ERRORS.get(code, 'unknown')}")
        self.code = code


def lib_path(plant: int = 0) -> str:
    name = "libpkv_oracle.so" if plant == 0 else f"libpkv_oracle_plant{plant}.so"
    return os.path.join(HERE, name)


def build(plant: int = 0, out: Optional[str] = None) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    out = out or lib_path(plant)
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           f"-DPKV_ORACLE_PLANT={plant}", SOURCE, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_LIBS = {}


def _load(plant: int = 0) -> ctypes.CDLL:
    if plant in _LIBS:
        return _LIBS[plant]
    path = lib_path(plant)
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SOURCE):
        build(plant)
    lib = ctypes.CDLL(path)
    P, I32, I64, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.pkv_oracle_store.argtypes = [P, P, P, I64, P, I64, P, I32, I32, I32, I32]
    lib.pkv_oracle_decode.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F]
    lib.pkv_oracle_prefill.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F]
    for fn in (lib.pkv_oracle_store, lib.pkv_oracle_decode, lib.pkv_oracle_prefill):
        fn.restype = ctypes.c_int
    lib.pkv_oracle_plant.restype = ctypes.c_int
    lib.pkv_oracle_threads.restype = ctypes.c_int
    _LIBS[plant] = lib
    return lib


def _bits(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit patterns of a CPU bf16 tensor as a C-contiguous uint16 array."""
    assert t.dtype == torch.bfloat16 and t.device.type == "cpu"
    return np.ascontiguousarray(t.contiguous().view(torch.int16).numpy()).view(np.uint16)


def _i32(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


class Oracle:
    """Handle on one build of the oracle (``plant`` selects a planted-mistake build)."""

    def __init__(self, plant: int = 0):
        self.plant = plant
        self.lib = _load(plant)

    def threads(self) -> int:
        """OpenMP threads the oracle's parallel loops use."""
        return int(self.lib.pkv_oracle_threads())

    # -- store --------------------------------------------------------------
    def store(self, k_cache: torch.Tensor, v_cache: torch.Tensor, key: torch.Tensor,
              value: torch.Tensor, slot_mapping) -> None:
        """In place: rows slot_mapping[i] of the caches become key[i] / value[i].

        k_cache/v_cache: CPU bf16 [num_blocks, block_size, H_kv, d] (contiguous);
        key/value: CPU bf16 [N, H_kv, d] whose last two dims are contiguous.
        """
        assert k_cache.is_contiguous() and v_cache.is_contiguous()
        nb, bs, H, d = k_cache.shape
        row = H * d
        kc = k_cache.view(torch.int16).numpy().view(np.uint16)  # shares memory
        vc = v_cache.view(torch.int16).numpy().view(np.uint16)
        N = key.shape[0]
        kin = _bits(key.reshape(N, row))
        vin = _bits(value.reshape(N, row))
        slots = _i32(slot_mapping)
        assert slots.shape == (N,)
        rc = self.lib.pkv_oracle_store(_ptr(kc), _ptr(vc), _ptr(kin), row, _ptr(vin), row,
                                       _ptr(slots), N, nb, bs, row)
        if rc:
            raise OracleError(rc)

    # -- attention ----------------------------------------------------------
    def decode(self, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
               block_tables, context_lens, softmax_scale: float) -> torch.Tensor:
        B, H_q, d = q.shape
        nb, bs, H_kv, d2 = k_cache.shape
        assert d2 == d
        bt = _i32(block_tables)
        maxb = bt.shape[1] if bt.ndim == 2 else 0
        cl = _i32(context_lens)
        qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
        out = np.zeros((B, H_q, d), dtype=np.float64)
        rc = self.lib.pkv_oracle_decode(_ptr(out), _ptr(qb), _ptr(kb), _ptr(vb), _ptr(bt),
                                        _ptr(cl), B, H_q, H_kv, d, nb, bs, maxb,
                                        float(softmax_scale))
        if rc:
            raise OracleError(rc)
        return torch.from_numpy(out)

    def prefill(self, q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                block_tables, cu_seqlens_q, cu_seqlens_k, softmax_scale: float) -> torch.Tensor:
        T, H_q, d = q.shape
        nb, bs, H_kv, d2 = k_cache.shape
        assert d2 == d
        bt = _i32(block_tables)
        maxb = bt.shape[1] if bt.ndim == 2 else 0
        cq, ck = _i32(cu_seqlens_q), _i32(cu_seqlens_k)
        B = cq.shape[0] - 1
        assert cq[-1] == T
        qb, kb, vb = _bits(q), _bits(k_cache), _bits(v_cache)
        out = np.zeros((T, H_q, d), dtype=np.float64)
        rc = self.lib.pkv_oracle_prefill(_ptr(out), _ptr(qb), _ptr(kb), _ptr(vb), _ptr(bt),
                                         _ptr(cq), _ptr(ck), B, H_q, H_kv, d, nb, bs, maxb,
                                         float(softmax_scale))
        if rc:
            raise OracleError(rc)
        return torch.from_numpy(out)


    def prefill_packed(self, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q,
                       cu_seqlens_k, softmax_scale: float) -> torch.Tensor:
        """Varlen causal prefill over packed K/V [total_k, H_kv, d]: key j of
        sequence b is token row cu_seqlens_k[b] + j (devpress page, the varlen
        call without a block table).  The same attention as prefill(), read
        through a one-token-per-block table that maps key j of sequence b to
        row cu_seqlens_k[b] + j."""
        total_k, H_kv, d = k.shape
        ck = _i32(cu_seqlens_k)
        B = ck.shape[0] - 1
        nk = ck[1:] - ck[:-1]
        width = max(1, int(nk.max()) if B > 0 else 1)
        table = np.full((max(B, 0), width), -1, dtype=np.int32)
        for b in range(B):
            table[b, : nk[b]] = np.arange(ck[b], ck[b + 1], dtype=np.int32)
        kc = k.contiguous().reshape(total_k, 1, H_kv, d)
        vc = v.contiguous().reshape(total_k, 1, H_kv, d)
        return self.prefill(q.contiguous(), kc, vc, table, cu_seqlens_q, cu_seqlens_k,
                            softmax_scale)


_DEFAULT: Optional[Oracle] = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle(0)
    return _DEFAULT


__all__ = ["Oracle", "OracleError", "build", "default", "prepare_decode", "prepare_prefill"]
