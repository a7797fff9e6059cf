"""ctypes loader for libpkv.so (the C ABI declared in include/pkv.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in the package.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpkv.so")

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_ELAUNCH, PKV_ESCRATCH = 0, 1, 2, 3, 4

# every symbol include/pkv.h declares
EXPORTS = (
    "pkv_status_string",
    "pkv_version",
    "pkv_prepare_metadata",
    "pkv_store",
    "pkv_decode_workspace_size",
    "pkv_decode",
    "pkv_store_decode",
    "pkv_prefill_varlen",
    "pkv_prefill_varlen_packed",
    "pkv_sample_workspace_size",
    "pkv_sample_gumbel",
    "pkv_sample_gumbel_noalloc",
    "pkv_pack_row_writes",
    "pkv_apply_row_writes",
    "pkv_prepare_metadata_device",
    "pkv_decode_graph_bucket",
    "pkv_decode_graph_create",
    "pkv_decode_graph_replay",
    "pkv_decode_step_run",
    "pkv_decode_graph_destroy",
)


class DecodeStep(ctypes.Structure):
    """Mirror of pkv_decode_step (include/pkv.h)."""
    _fields_ = [
        ("layers", ctypes.c_int32), ("max_batch", ctypes.c_int32),
        ("H_q", ctypes.c_int32), ("H_kv", ctypes.c_int32), ("d", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32), ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
        ("slot_mapping", ctypes.c_void_p), ("context_lens", ctypes.c_void_p),
        ("block_tables", ctypes.c_void_p),
        ("q", ctypes.POINTER(ctypes.c_void_p)), ("key", ctypes.POINTER(ctypes.c_void_p)),
        ("value", ctypes.POINTER(ctypes.c_void_p)),
        ("key_stride", ctypes.c_int64), ("value_stride", ctypes.c_int64),
        ("k_cache", ctypes.POINTER(ctypes.c_void_p)), ("v_cache", ctypes.POINTER(ctypes.c_void_p)),
        ("out", ctypes.POINTER(ctypes.c_void_p)),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
    ]


class PkvError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed: {message} (status {status})")
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_110_amd.build` "
            "(hipcc, gfx950). There is no CPU fallback."
        )
    lib = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F, SZ = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                          ctypes.c_size_t)
    lib.pkv_status_string.argtypes = [ctypes.c_int]
    lib.pkv_status_string.restype = ctypes.c_char_p
    lib.pkv_version.argtypes = []
    lib.pkv_version.restype = ctypes.c_int
    lib.pkv_prepare_metadata.argtypes = [I32, P, P, P, P, I32, I32, P, P, P, P, P, P, P]
    lib.pkv_prepare_metadata.restype = ctypes.c_int
    lib.pkv_store.argtypes = [P, I64, P, I64, P, P, P, I32, I32, I32, I32, I32, P]
    lib.pkv_store.restype = ctypes.c_int
    lib.pkv_decode_workspace_size.argtypes = [I32, I32, I32, I32, I32, I32]
    lib.pkv_decode_workspace_size.restype = SZ
    lib.pkv_decode.argtypes = [P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32, F, P, SZ, P]
    lib.pkv_decode.restype = ctypes.c_int
    lib.pkv_store_decode.argtypes = [P, P, P, I64, P, I64, P, P, P, P, I32, I32, I32, I32, I32,
                                     I32, I32, F, P, SZ, P]
    lib.pkv_store_decode.restype = ctypes.c_int
    lib.pkv_prefill_varlen.argtypes = [P, P, P, P, P, P, P, I32, I32, I32, I32, I32, I32, I32,
                                       I32, I32, I32, F, P]
    lib.pkv_prefill_varlen.restype = ctypes.c_int
    lib.pkv_prefill_varlen_packed.argtypes = [P, P, I64, P, I64, P, I64, P, P, I32, I32, I32, I32,
                                              I32, I32, I32, I32, F, P]
    lib.pkv_prefill_varlen_packed.restype = ctypes.c_int
    lib.pkv_sample_workspace_size.argtypes = [I32, I32]
    lib.pkv_sample_workspace_size.restype = SZ
    lib.pkv_sample_gumbel.argtypes = [P, P, I32, I64, I32, I32, P, P, P, P, SZ, P]
    lib.pkv_sample_gumbel.restype = ctypes.c_int
    lib.pkv_sample_gumbel_noalloc.argtypes = [P, P, I32, I64, I32, I32, P, P, P, P]
    lib.pkv_sample_gumbel_noalloc.restype = ctypes.c_int
    lib.pkv_pack_row_writes.argtypes = [I32, P, P, P, P, I32, I32, P, I64, P]
    lib.pkv_pack_row_writes.restype = ctypes.c_int
    lib.pkv_apply_row_writes.argtypes = [P, I64, I32, I32, P, I32, I32, P]
    lib.pkv_apply_row_writes.restype = ctypes.c_int
    lib.pkv_prepare_metadata_device.argtypes = [I32, P, P, P, P, I32, I64, I32, I32, I32, P, P, P,
                                                P, P, P, P, P]
    lib.pkv_prepare_metadata_device.restype = ctypes.c_int
    SP = ctypes.POINTER(DecodeStep)
    lib.pkv_decode_graph_bucket.argtypes = [I32, I32]
    lib.pkv_decode_graph_bucket.restype = I32
    lib.pkv_decode_graph_create.argtypes = [SP, ctypes.POINTER(P)]
    lib.pkv_decode_graph_create.restype = ctypes.c_int
    lib.pkv_decode_graph_replay.argtypes = [P, I32, P]
    lib.pkv_decode_graph_replay.restype = ctypes.c_int
    lib.pkv_decode_step_run.argtypes = [SP, I32, P]
    lib.pkv_decode_step_run.restype = ctypes.c_int
    lib.pkv_decode_graph_destroy.argtypes = [P]
    lib.pkv_decode_graph_destroy.restype = None
    _lib = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != PKV_OK:
        msg = load().pkv_status_string(status).decode()
        raise PkvError(fn, status, msg)
