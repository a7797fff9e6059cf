"""Paged-KV attention for AMD MI355X (gfx950): Python binding of libpkv.

Thin marshalling over the C ABI in include/pkv.h: every function checks the
torch tensors it is given (device, dtype, shape, contiguity), turns them into
raw pointers and sizes, and calls the library on the current HIP stream.  All
computation happens in the library's kernels (or, for ``prepare_metadata``,
in its host routine).  Output and workspace tensors are allocated with torch
when the caller does not pass them.

Functions:
    prepare_metadata(seqs, block_size, max_blocks_per_seq) -> dict (host int32 tensors)
    store(key, value, k_cache, v_cache, slot_mapping)
    decode(q, k_cache, v_cache, block_tables, context_lens, softmax_scale=None, ...)
    prefill_varlen(q, k_cache, v_cache, block_tables, cu_seqlens_q, cu_seqlens_k,
                   max_seqlen_q, max_seqlen_k, softmax_scale=None, ...)
    prefill_varlen_packed(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, ...)
    pack_row_writes(writes, num_rows, num_cols) -> host int32 tensor
    apply_row_writes(table, packed, num_writes, total)
    StagedWrites(table): stage_write(row, start, values), apply()
    prepare_metadata_device(idx_mapping, num_computed, num_scheduled, block_table, ...) -> dict
    sample_gumbel(logits, seeds, temperatures=None, offsets=None) -> int64 tokens
    sample_gumbel_noalloc(logits, seeds, temperatures=None, offsets=None, out=None) -> int64 tokens
    graph_bucket(max_batch, batch) -> int
    DecodeGraph(k_caches, v_caches, max_batch, H_q, max_blocks_per_seq, ...)
"""
from __future__ import annotations

import contextlib
import ctypes
import math
from typing import Optional, Sequence

import torch

from ._lib import EXPORTS, LIB_PATH, DecodeStep, PkvError, check, load

__all__ = [
    "prepare_metadata", "store", "decode", "store_decode", "decode_workspace_size", "prefill_varlen",
    "prefill_varlen_packed", "pack_row_writes", "apply_row_writes", "StagedWrites",
    "prepare_metadata_device", "sample_gumbel", "sample_gumbel_noalloc", "sample_workspace_size",
    "graph_bucket", "DecodeGraph", "PkvError", "LIB_PATH", "EXPORTS",
    "version",
]


def version() -> int:
    return load().pkv_version()


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _dev_i32(t: torch.Tensor, name: str) -> None:
    _need(t.is_cuda and t.dtype == torch.int32 and t.is_contiguous(),
          f"{name} must be a contiguous int32 GPU tensor")


def _cache_geometry(k_cache: torch.Tensor, v_cache: torch.Tensor):
    _need(k_cache.dim() == 4 and k_cache.shape == v_cache.shape,
          "k_cache/v_cache must both be [num_blocks, block_size, H_kv, d]")
    _need(k_cache.dtype == torch.bfloat16 and v_cache.dtype == torch.bfloat16,
          "caches must be bfloat16")
    _need(k_cache.is_cuda and v_cache.is_cuda, "caches must be GPU tensors")
    _need(k_cache.is_contiguous() and v_cache.is_contiguous(), "caches must be contiguous")
    return tuple(int(x) for x in k_cache.shape)


def prepare_metadata(seqs: Sequence, block_size: int, max_blocks_per_seq: int) -> dict:
    """Host metadata of one step from per-sequence block-manager state.

    ``seqs``: objects with ``block_ids`` (physical ids, logical order),
    ``num_cached`` and ``num_new``.  Returns CPU int32 tensors ``slot_mapping``,
    ``context_lens``, ``cu_seqlens_q``, ``cu_seqlens_k``, ``block_tables`` and
    the ints ``max_seqlen_q``/``max_seqlen_k``.
    """
    lib = load()
    B = len(seqs)
    cached = torch.tensor([s.num_cached for s in seqs], dtype=torch.int32)
    new = torch.tensor([s.num_new for s in seqs], dtype=torch.int32)
    offs = [0]
    for s in seqs:
        offs.append(offs[-1] + len(s.block_ids))
    offsets = torch.tensor(offs, dtype=torch.int32)
    ids = torch.tensor([b for s in seqs for b in s.block_ids] or [0], dtype=torch.int32)
    total_new = int(new.sum()) if B else 0
    slot = torch.empty(max(total_new, 1), dtype=torch.int32)
    ctx = torch.empty(max(B, 1), dtype=torch.int32)
    cu_q = torch.empty(B + 1, dtype=torch.int32)
    cu_k = torch.empty(B + 1, dtype=torch.int32)
    bt = torch.empty(max(B * max_blocks_per_seq, 1), dtype=torch.int32)
    mq, mk = ctypes.c_int32(0), ctypes.c_int32(0)
    check("pkv_prepare_metadata", lib.pkv_prepare_metadata(
        B, _ptr(cached), _ptr(new), _ptr(offsets), _ptr(ids), block_size, max_blocks_per_seq,
        _ptr(slot), _ptr(ctx), _ptr(cu_q), _ptr(cu_k), _ptr(bt), ctypes.byref(mq),
        ctypes.byref(mk)))
    return dict(
        slot_mapping=slot[:total_new], context_lens=ctx[:B], cu_seqlens_q=cu_q,
        cu_seqlens_k=cu_k, block_tables=bt[: B * max_blocks_per_seq].view(B, max_blocks_per_seq),
        max_seqlen_q=mq.value, max_seqlen_k=mk.value,
    )


def store(key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
          slot_mapping: torch.Tensor, stream=None) -> None:
    """k_cache/v_cache row slot_mapping[i] <- key[i]/value[i]; slot -1 is skipped."""
    nb, bs, H_kv, d = _cache_geometry(k_cache, v_cache)
    _need(key.dim() == 3 and key.shape == value.shape and tuple(key.shape[1:]) == (H_kv, d),
          "key/value must be [N, H_kv, d] matching the cache")
    _need(key.dtype == torch.bfloat16 and value.dtype == torch.bfloat16, "key/value bfloat16")
    _need(key.is_cuda and value.is_cuda, "key/value must be GPU tensors")
    _need(key.stride(2) == 1 and key.stride(1) == d and value.stride(2) == 1
          and value.stride(1) == d, "key/value head and d dims must be contiguous")
    _dev_i32(slot_mapping, "slot_mapping")
    N = key.shape[0]
    _need(slot_mapping.shape == (N,), "slot_mapping must be [N]")
    check("pkv_store", load().pkv_store(
        _ptr(key), key.stride(0), _ptr(value), value.stride(0), _ptr(k_cache), _ptr(v_cache),
        _ptr(slot_mapping), N, nb, bs, H_kv, d, _stream(stream)))


def decode_workspace_size(B: int, H_q: int, H_kv: int, d: int, block_size: int,
                          max_blocks_per_seq: int) -> int:
    return int(load().pkv_decode_workspace_size(B, H_q, H_kv, d, block_size, max_blocks_per_seq))


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           block_tables: torch.Tensor, context_lens: torch.Tensor,
           softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
           workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Paged decode attention; q [B, H_q, d] -> out [B, H_q, d] (bf16)."""
    nb, bs, H_kv, d = _cache_geometry(k_cache, v_cache)
    _need(q.dim() == 3 and q.shape[2] == d and q.dtype == torch.bfloat16 and q.is_cuda
          and q.is_contiguous(), "q must be a contiguous bf16 GPU tensor [B, H_q, d]")
    B, H_q = int(q.shape[0]), int(q.shape[1])
    _dev_i32(block_tables, "block_tables")
    _dev_i32(context_lens, "context_lens")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B, maxb]")
    _need(context_lens.shape == (B,), "context_lens must be [B]")
    maxb = int(block_tables.shape[1])
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous(), "bad out")
    ws_bytes = decode_workspace_size(B, H_q, H_kv, d, bs, maxb)
    if workspace is None and ws_bytes > 0:
        workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=q.device)
    have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    check("pkv_decode", load().pkv_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        B, H_q, H_kv, d, nb, bs, maxb, scale, _ptr(workspace), have, _stream(stream)))
    return out


def store_decode(q: torch.Tensor, key: torch.Tensor, value: torch.Tensor, k_cache: torch.Tensor,
                 v_cache: torch.Tensor, block_tables: torch.Tensor, context_lens: torch.Tensor,
                 softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """The decode step's store fused into its attention: key/value [B, H_kv, d] (sequence
    b's new token, stored at position context_lens[b] - 1) and q [B, H_q, d] -> out."""
    nb, bs, H_kv, d = _cache_geometry(k_cache, v_cache)
    _need(q.dim() == 3 and q.shape[2] == d and q.dtype == torch.bfloat16 and q.is_cuda
          and q.is_contiguous(), "q must be a contiguous bf16 GPU tensor [B, H_q, d]")
    B, H_q = int(q.shape[0]), int(q.shape[1])
    _need(key.dim() == 3 and key.shape == value.shape and tuple(key.shape) == (B, H_kv, d),
          "key/value must be [B, H_kv, d] matching q and the cache")
    _need(key.dtype == torch.bfloat16 and value.dtype == torch.bfloat16, "key/value bfloat16")
    _need(key.is_cuda and value.is_cuda, "key/value must be GPU tensors")
    _need(key.stride(2) == 1 and key.stride(1) == d and value.stride(2) == 1
          and value.stride(1) == d, "key/value head and d dims must be contiguous")
    _dev_i32(block_tables, "block_tables")
    _dev_i32(context_lens, "context_lens")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B, maxb]")
    _need(context_lens.shape == (B,), "context_lens must be [B]")
    maxb = int(block_tables.shape[1])
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous(), "bad out")
    ws_bytes = decode_workspace_size(B, H_q, H_kv, d, bs, maxb)
    if workspace is None and ws_bytes > 0:
        workspace = torch.zeros(ws_bytes, dtype=torch.uint8, device=q.device)
    have = 0 if workspace is None else workspace.numel() * workspace.element_size()
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    check("pkv_store_decode", load().pkv_store_decode(
        _ptr(out), _ptr(q), _ptr(key), key.stride(0), _ptr(value), value.stride(0),
        _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        B, H_q, H_kv, d, nb, bs, maxb, scale, _ptr(workspace), have, _stream(stream)))
    return out

def prefill_varlen(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   block_tables: torch.Tensor, cu_seqlens_q: torch.Tensor,
                   cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int,
                   softmax_scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                   stream=None) -> torch.Tensor:
    """Varlen causal prefill over the paged cache; q [total_q, H_q, d] -> out (bf16)."""
    nb, bs, H_kv, d = _cache_geometry(k_cache, v_cache)
    _need(q.dim() == 3 and q.shape[2] == d and q.dtype == torch.bfloat16 and q.is_cuda
          and q.is_contiguous(), "q must be a contiguous bf16 GPU tensor [total_q, H_q, d]")
    total_q, H_q = int(q.shape[0]), int(q.shape[1])
    _dev_i32(block_tables, "block_tables")
    _dev_i32(cu_seqlens_q, "cu_seqlens_q")
    _dev_i32(cu_seqlens_k, "cu_seqlens_k")
    B = int(cu_seqlens_q.shape[0]) - 1
    _need(cu_seqlens_k.shape == cu_seqlens_q.shape and B >= 0, "cu_seqlens must be [B+1]")
    _need(block_tables.dim() == 2 and block_tables.shape[0] == B, "block_tables must be [B, maxb]")
    if out is None:
        out = torch.empty_like(q)
    _need(out.shape == q.shape and out.dtype == q.dtype and out.is_contiguous(), "bad out")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    check("pkv_prefill_varlen", load().pkv_prefill_varlen(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_k), B, total_q, int(max_seqlen_q), int(max_seqlen_k), H_q, H_kv, d, nb, bs,
        int(block_tables.shape[1]), scale, _stream(stream)))
    return out


def _rows(t: torch.Tensor, name: str, H: int, d: int) -> None:
    _need(t.dim() == 3 and tuple(t.shape[1:]) == (H, d) and t.dtype == torch.bfloat16
          and t.is_cuda, f"{name} must be a bf16 GPU tensor [tokens, {H}, {d}]")
    _need(t.stride(2) == 1 and t.stride(1) == d, f"{name}: head and d dims must be contiguous")


def prefill_varlen_packed(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                          cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                          max_seqlen_q: int, max_seqlen_k: int,
                          softmax_scale: Optional[float] = None,
                          out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Varlen causal prefill over packed K/V [total_k, H_kv, d] (token rows of all
    sequences stacked, addressed by cu_seqlens_k); q [total_q, H_q, d] -> out (bf16).
    q, k and v may be row-strided views (e.g. of a fused QKV projection)."""
    _need(q.dim() == 3 and k.dim() == 3, "q/k/v must be [tokens, heads, d]")
    H_q, d = int(q.shape[1]), int(q.shape[2])
    H_kv = int(k.shape[1])
    _rows(q, "q", H_q, d)
    _rows(k, "k", H_kv, d)
    _rows(v, "v", H_kv, d)
    _need(v.shape[0] == k.shape[0], "k and v must have the same number of rows")
    _dev_i32(cu_seqlens_q, "cu_seqlens_q")
    _dev_i32(cu_seqlens_k, "cu_seqlens_k")
    B = int(cu_seqlens_q.shape[0]) - 1
    _need(cu_seqlens_k.shape == cu_seqlens_q.shape and B >= 0, "cu_seqlens must be [B+1]")
    total_q, total_k = int(q.shape[0]), int(k.shape[0])
    if out is None:
        out = torch.empty((total_q, H_q, d), dtype=q.dtype, device=q.device)
    _need(out.shape == (total_q, H_q, d) and out.dtype == q.dtype and out.is_contiguous(),
          "bad out")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    check("pkv_prefill_varlen_packed", load().pkv_prefill_varlen_packed(
        _ptr(out), _ptr(q), q.stride(0), _ptr(k), k.stride(0), _ptr(v), v.stride(0),
        _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, total_q, total_k, int(max_seqlen_q),
        int(max_seqlen_k), H_q, H_kv, d, scale, _stream(stream)))
    return out


def _host_i32(values) -> torch.Tensor:
    return torch.as_tensor(values, dtype=torch.int32).contiguous()


def pack_row_writes(writes, num_rows: int, num_cols: int, pin: bool = False) -> torch.Tensor:
    """Packs ragged writes ``[(row, start, values), ...]`` for a [num_rows, num_cols]
    table into one host int32 buffer (layout in include/pkv.h); ``pin`` puts it in
    pinned memory for an asynchronous copy."""
    n = len(writes)
    rows = _host_i32([w[0] for w in writes] or [0])
    starts = _host_i32([w[1] for w in writes] or [0])
    lens = _host_i32([len(w[2]) for w in writes] or [0])
    flat = [int(v) for w in writes for v in w[2]]
    values = _host_i32(flat or [0])
    size = 3 * n + 1 + len(flat)
    packed = torch.empty(size, dtype=torch.int32, pin_memory=pin)
    got = ctypes.c_int64(0)
    check("pkv_pack_row_writes", load().pkv_pack_row_writes(
        n, _ptr(rows), _ptr(starts), _ptr(lens), _ptr(values), int(num_rows), int(num_cols),
        _ptr(packed), size, ctypes.byref(got)))
    return packed


def apply_row_writes(table: torch.Tensor, packed: torch.Tensor, num_writes: int, total: int,
                     stream=None) -> None:
    """Applies a packed buffer (device int32) to a device int32 table [rows, cols]."""
    _need(table.is_cuda and table.dtype == torch.int32 and table.dim() == 2
          and table.stride(1) == 1, "table must be a GPU int32 [rows, cols] tensor, cols contiguous")
    _dev_i32(packed, "packed")
    _need(packed.numel() >= 3 * num_writes + 1 + total, "packed buffer too small")
    check("pkv_apply_row_writes", load().pkv_apply_row_writes(
        _ptr(table), table.stride(0), int(table.shape[0]), int(table.shape[1]), _ptr(packed),
        int(num_writes), int(total), _stream(stream)))


class StagedWrites:
    """Ragged writes into a device int32 table, staged on the host and applied
    in one kernel (pkv_pack_row_writes + pkv_apply_row_writes).  Each apply packs
    into fresh pinned memory, so staging the next writes never races the copy of
    the previous ones."""

    def __init__(self, table: torch.Tensor):
        _need(table.is_cuda and table.dtype == torch.int32 and table.dim() == 2,
              "table must be a GPU int32 [rows, cols] tensor")
        self.table = table
        self.pending = []

    def stage_write(self, row: int, start: int, values) -> None:
        self.pending.append((int(row), int(start), [int(v) for v in values]))

    def apply(self, stream: Optional[torch.cuda.Stream] = None) -> None:
        """Packs, copies and applies every staged write on ``stream`` (default:
        the current stream)."""
        if not self.pending:
            return
        writes, self.pending = self.pending, []
        packed = pack_row_writes(writes, self.table.shape[0], self.table.shape[1], pin=True)
        with torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext():
            dev = packed.to(self.table.device, non_blocking=True)
            total = sum(len(w[2]) for w in writes)
            apply_row_writes(self.table, dev, len(writes), total)


def prepare_metadata_device(idx_mapping: Optional[torch.Tensor], num_computed: torch.Tensor,
                            num_scheduled: torch.Tensor, block_table: torch.Tensor,
                            block_size: int, max_blocks_per_seq: int, max_tokens: int,
                            positions: bool = True, block_tables: bool = True,
                            out: Optional[dict] = None, stream=None) -> dict:
    """Step metadata built on the device from request state kept on the device
    (pkv_prepare_metadata_device).  Returns device tensors ``cu_seqlens_q``,
    ``cu_seqlens_k``, ``context_lens``, ``slot_mapping`` [max_tokens],
    ``positions`` [max_tokens] int64, ``block_tables`` [B, max_blocks_per_seq] and
    ``max_seqlens`` [2]; ``out`` may supply any of them (e.g. a graph's static
    buffers)."""
    _dev_i32(num_computed, "num_computed")
    _dev_i32(num_scheduled, "num_scheduled")
    _need(block_table.is_cuda and block_table.dtype == torch.int32 and block_table.dim() == 2
          and block_table.stride(1) == 1, "block_table must be a GPU int32 [reqs, width] tensor")
    if idx_mapping is not None:
        _dev_i32(idx_mapping, "idx_mapping")
    B = int(num_scheduled.shape[0])
    dev = num_scheduled.device
    out = dict(out or {})

    def buf(name, shape, dtype):
        if name not in out:
            out[name] = torch.empty(shape, dtype=dtype, device=dev)
        t = out[name]
        _need(t.is_cuda and t.dtype == dtype and t.is_contiguous() and t.numel() >= math.prod(shape),
              f"bad {name}")
        return t

    cq = buf("cu_seqlens_q", (B + 1,), torch.int32)
    ck = buf("cu_seqlens_k", (B + 1,), torch.int32)
    ctx = buf("context_lens", (max(B, 1),), torch.int32)
    slots = buf("slot_mapping", (max(max_tokens, 1),), torch.int32)
    pos = buf("positions", (max(max_tokens, 1),), torch.int64) if positions else None
    bt = buf("block_tables", (B, max_blocks_per_seq), torch.int32) if block_tables else None
    mx = buf("max_seqlens", (2,), torch.int32)
    check("pkv_prepare_metadata_device", load().pkv_prepare_metadata_device(
        B, _ptr(idx_mapping), _ptr(num_computed), _ptr(num_scheduled), _ptr(block_table),
        int(block_table.shape[0]), block_table.stride(0), int(block_size), int(max_blocks_per_seq),
        int(max_tokens), _ptr(cq), _ptr(ck), _ptr(ctx), _ptr(pos), _ptr(slots), _ptr(bt), _ptr(mx),
        _stream(stream)))
    return out


def sample_workspace_size(B: int, V: int) -> int:
    return int(load().pkv_sample_workspace_size(int(B), int(V)))


def sample_gumbel(logits: torch.Tensor, seeds: torch.Tensor,
                  temperatures: Optional[torch.Tensor] = None,
                  offsets: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Gumbel-max sampling (pkv_sample_gumbel): one token per row of ``logits``
    [B, V] (bf16 or fp32, unit stride along V), drawn from softmax(logits / T)
    with Philox noise keyed by ``seeds`` [B] int64 and counted by ``offsets``
    [B] int64; T <= 0 picks the argmax.  Returns int64 tokens [B]."""
    _need(logits.is_cuda and logits.dim() == 2 and logits.stride(1) == 1
          and logits.dtype in (torch.bfloat16, torch.float32),
          "logits must be a GPU bf16/fp32 [B, V] tensor with unit stride along V")
    B, V = int(logits.shape[0]), int(logits.shape[1])
    _need(seeds.is_cuda and seeds.dtype == torch.int64 and seeds.shape == (B,)
          and seeds.is_contiguous(), "seeds must be a contiguous GPU int64 [B] tensor")
    if offsets is not None:
        _need(offsets.is_cuda and offsets.dtype == torch.int64 and offsets.shape == (B,)
              and offsets.is_contiguous(), "offsets must be a contiguous GPU int64 [B] tensor")
    if temperatures is not None:
        _need(temperatures.is_cuda and temperatures.dtype == torch.float32
              and temperatures.shape == (B,) and temperatures.is_contiguous(),
              "temperatures must be a contiguous GPU fp32 [B] tensor")
    if out is None:
        out = torch.empty(B, dtype=torch.int64, device=logits.device)
    _need(out.dtype == torch.int64 and out.shape == (B,) and out.is_contiguous(), "bad out")
    need = sample_workspace_size(B, V)
    if workspace is None:
        workspace = torch.empty(max(need, 8), dtype=torch.uint8, device=logits.device)
    have = workspace.numel() * workspace.element_size()
    check("pkv_sample_gumbel", load().pkv_sample_gumbel(
        _ptr(out), _ptr(logits), int(logits.dtype == torch.bfloat16), logits.stride(0), B, V,
        _ptr(temperatures), _ptr(seeds), _ptr(offsets), _ptr(workspace), have, _stream(stream)))
    return out


def sample_gumbel_noalloc(logits: torch.Tensor, seeds: torch.Tensor,
                          temperatures: Optional[torch.Tensor] = None,
                          offsets: Optional[torch.Tensor] = None,
                          out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """sample_gumbel without a workspace (pkv_sample_gumbel_noalloc): the
    library's fixed per-device scratch holds the chunk keys.  Pass ``out`` to
    allocate nothing at all.  Returns int64 tokens [B]."""
    _need(logits.is_cuda and logits.dim() == 2 and logits.stride(1) == 1
          and logits.dtype in (torch.bfloat16, torch.float32),
          "logits must be a GPU bf16/fp32 [B, V] tensor with unit stride along V")
    B, V = int(logits.shape[0]), int(logits.shape[1])
    _need(seeds.is_cuda and seeds.dtype == torch.int64 and seeds.shape == (B,)
          and seeds.is_contiguous(), "seeds must be a contiguous GPU int64 [B] tensor")
    if offsets is not None:
        _need(offsets.is_cuda and offsets.dtype == torch.int64 and offsets.shape == (B,)
              and offsets.is_contiguous(), "offsets must be a contiguous GPU int64 [B] tensor")
    if temperatures is not None:
        _need(temperatures.is_cuda and temperatures.dtype == torch.float32
              and temperatures.shape == (B,) and temperatures.is_contiguous(),
              "temperatures must be a contiguous GPU fp32 [B] tensor")
    if out is None:
        out = torch.empty(B, dtype=torch.int64, device=logits.device)
    _need(out.dtype == torch.int64 and out.shape == (B,) and out.is_contiguous(), "bad out")
    check("pkv_sample_gumbel_noalloc", load().pkv_sample_gumbel_noalloc(
        _ptr(out), _ptr(logits), int(logits.dtype == torch.bfloat16), logits.stride(0), B, V,
        _ptr(temperatures), _ptr(seeds), _ptr(offsets), _stream(stream)))
    return out


def graph_bucket(max_batch: int, batch: int) -> int:
    """Bucket a batch of ``batch`` rows replays in a graph set of ``max_batch``
    rows (-1 when there is none)."""
    return int(load().pkv_decode_graph_bucket(int(max_batch), int(batch)))


class DecodeGraph:
    """Graph-captured decode step with batch buckets (pkv_decode_graph_* in
    include/pkv.h): every layer's store + decode, one HIP graph per bucket.

    The static buffers, sized for ``max_batch`` rows, are allocated here with
    torch and filled by the caller before each step (rows ``[0, batch)``):
    ``slot_mapping``, ``context_lens``, ``block_tables``, ``q[l]``, ``key[l]``,
    ``value[l]`` (views of one fused ``kv_new[l]`` buffer, K then V per token).
    After ``replay(batch)`` (or ``run_eager(batch)``), ``out[l][:batch]`` holds
    layer l's attention output.  ``k_caches`` / ``v_caches`` are the per-layer
    cache tensors ``[num_blocks, block_size, H_kv, d]``; they must outlive the
    graphs.  Batches above ``max_batch`` are the caller's eager calls.
    """

    def __init__(self, k_caches, v_caches, max_batch: int, H_q: int, max_blocks_per_seq: int,
                 softmax_scale: Optional[float] = None):
        _need(len(k_caches) == len(v_caches) and len(k_caches) >= 1, "one k and v cache per layer")
        geo = _cache_geometry(k_caches[0], v_caches[0])
        for kc, vc in zip(k_caches, v_caches):
            _need(_cache_geometry(kc, vc) == geo, "every layer's caches must have one geometry")
        nb, bs, H_kv, d = geo
        L, dev = len(k_caches), k_caches[0].device
        self.layers, self.max_batch = L, int(max_batch)
        self.H_q, self.H_kv, self.d = int(H_q), H_kv, d
        self.k_caches, self.v_caches = list(k_caches), list(v_caches)
        mb = self.max_batch
        self.slot_mapping = torch.full((mb,), -1, dtype=torch.int32, device=dev)
        self.context_lens = torch.zeros(mb, dtype=torch.int32, device=dev)
        self.block_tables = torch.full((mb, max_blocks_per_seq), -1, dtype=torch.int32, device=dev)
        self.q = torch.zeros((L, mb, H_q, d), dtype=torch.bfloat16, device=dev)
        self.kv_new = torch.zeros((L, mb, 2 * H_kv * d), dtype=torch.bfloat16, device=dev)
        self.key = [self.kv_new[l, :, : H_kv * d].view(mb, H_kv, d) for l in range(L)]
        self.value = [self.kv_new[l, :, H_kv * d:].view(mb, H_kv, d) for l in range(L)]
        self.out = torch.zeros((L, mb, H_q, d), dtype=torch.bfloat16, device=dev)
        ws = decode_workspace_size(mb, H_q, H_kv, d, bs, max_blocks_per_seq)
        _need(ws > 0, "unsupported decode shape")
        self.workspace = torch.zeros(ws, dtype=torch.uint8, device=dev)
        arr = ctypes.c_void_p * L
        self._arrays = [
            arr(*[self.q[l].data_ptr() for l in range(L)]),
            arr(*[t.data_ptr() for t in self.key]),
            arr(*[t.data_ptr() for t in self.value]),
            arr(*[t.data_ptr() for t in self.k_caches]),
            arr(*[t.data_ptr() for t in self.v_caches]),
            arr(*[self.out[l].data_ptr() for l in range(L)]),
        ]
        aq, ak, av, akc, avc, ao = self._arrays
        scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
        self._step = DecodeStep(
            L, mb, self.H_q, H_kv, d, nb, bs, int(max_blocks_per_seq), scale,
            self.slot_mapping.data_ptr(), self.context_lens.data_ptr(),
            self.block_tables.data_ptr(), aq, ak, av, self.kv_new.stride(1),
            self.kv_new.stride(1), akc, avc, ao, self.workspace.data_ptr(), ws)
        handle = ctypes.c_void_p(0)
        check("pkv_decode_graph_create",
              load().pkv_decode_graph_create(ctypes.byref(self._step), ctypes.byref(handle)))
        self._handle = handle

    def bucket(self, batch: int) -> int:
        return graph_bucket(self.max_batch, batch)

    def replay(self, batch: int, stream=None) -> None:
        """Pads rows [batch, bucket) and replays the bucket's graph."""
        _need(self._handle is not None, "graphs already released")
        check("pkv_decode_graph_replay",
              load().pkv_decode_graph_replay(self._handle, int(batch), _stream(stream)))

    def run_eager(self, batch: int, stream=None) -> None:
        """The same step as individual launches over rows [0, batch)."""
        check("pkv_decode_step_run",
              load().pkv_decode_step_run(ctypes.byref(self._step), int(batch), _stream(stream)))

    def close(self) -> None:
        if getattr(self, "_handle", None) is not None:
            load().pkv_decode_graph_destroy(self._handle)
            self._handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
