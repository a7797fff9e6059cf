"""Shared steps of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on host copies of the same inputs, compare."""
from __future__ import annotations

import math
import sys

import torch

import oracle as O
import paged_kv_cache_110_amd as pkv
from workloads import Tensors

TOL = 1e-2  # max-abs error bound for bf16 attention outputs against the float64 oracle


def bound(ref: torch.Tensor, tol: float = TOL) -> torch.Tensor:
    """Per-element error bound: ``tol``, except where a bf16 output cannot meet it.

    Outputs are bf16 (round to nearest even).  Below |o| = 4 the bf16 spacing is
    at most 2^-6, so rounding costs at most 2^-7 < 1e-2 and the bar is ``tol``.
    From |o| = 4 up the spacing is 2^-5 or more, and no bf16 value can be within
    1e-2 of every real; there the bar is half a bf16 spacing of the reference plus
    2e-3 for the fp32 arithmetic and the bf16 rounding of P before the PV product.
    """
    mag = ref.abs().clamp_min(1e-30)
    half_spacing = torch.exp2(torch.floor(torch.log2(mag)) - 8)
    return torch.where(mag < 4, torch.full_like(ref, tol), torch.maximum(half_spacing + 2e-3, torch.full_like(ref, tol)))


def log(msg: str) -> None:
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def scale_of(d: int) -> float:
    return 1.0 / math.sqrt(d)


def cpu_copy(t: Tensors, layers=None) -> Tensors:
    if layers is None:
        pool = t.pool.cpu()
    else:
        pool = torch.stack([t.pool[:, layer].cpu() for layer in layers], dim=1)
    return Tensors(pool=pool, q=t.q.cpu(), kv_new=t.kv_new.cpu(), H_kv=t.H_kv, d=t.d)


def device_meta(meta: dict, device) -> dict:
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in meta.items()}


def gpu_store(plan, tens: Tensors, dmeta: dict, layer: int = 0) -> None:
    pkv.store(tens.k_new(layer), tens.v_new(layer), tens.k_cache(layer), tens.v_cache(layer),
              dmeta["slot_mapping"])


def gpu_attention(plan, tens: Tensors, dmeta: dict, layer: int = 0) -> torch.Tensor:
    kc, vc = tens.k_cache(layer), tens.v_cache(layer)
    if plan.kind == "decode":
        return pkv.decode(tens.q[layer], kc, vc, dmeta["block_tables"], dmeta["context_lens"],
                          scale_of(plan.d))
    return pkv.prefill_varlen(tens.q[layer], kc, vc, dmeta["block_tables"],
                              dmeta["cu_seqlens_q"], dmeta["cu_seqlens_k"],
                              dmeta["max_seqlen_q"], dmeta["max_seqlen_k"], scale_of(plan.d))


def oracle_meta(plan) -> dict:
    if plan.kind == "decode":
        m = O.prepare_decode(plan.seqs, plan.block_size, plan.max_blocks_per_seq)
        m.update(O.prepare_prefill(plan.seqs, plan.block_size, plan.max_blocks_per_seq))
        return m
    return O.prepare_prefill(plan.seqs, plan.block_size, plan.max_blocks_per_seq)


def oracle_store(host: Tensors, meta: dict, layer: int = 0) -> None:
    O.default().store(host.k_cache(layer), host.v_cache(layer), host.k_new(layer),
                      host.v_new(layer), meta["slot_mapping"])


def oracle_attention(plan, host: Tensors, meta: dict, layer: int = 0, q_layer=None):
    q = host.q[layer if q_layer is None else q_layer]
    if plan.kind == "decode":
        return O.default().decode(q, host.k_cache(layer), host.v_cache(layer),
                                  meta["block_tables"], meta["context_lens"], scale_of(plan.d))
    return O.default().prefill(q, host.k_cache(layer), host.v_cache(layer), meta["block_tables"],
                               meta["cu_seqlens_q"], meta["cu_seqlens_k"], scale_of(plan.d))


def assert_close(got: torch.Tensor, ref: torch.Tensor, what: str, tol: float = TOL) -> float:
    g = got.detach().float().cpu().double()
    assert torch.isfinite(g).all(), f"{what}: non-finite GPU output"
    assert torch.isfinite(ref).all(), f"{what}: non-finite oracle output"
    diff = (g - ref).abs()
    err = diff.max().item() if g.numel() else 0.0
    big = int((ref.abs() >= 4).sum())
    log(f"{what}: max abs err {err:.3e} over {g.numel()} values ({big} with |o| >= 4)")
    over = diff > bound(ref, tol)
    assert not over.any(), (f"{what}: {int(over.sum())} values beyond the bound, worst "
                            f"{diff[over].max().item()} at |o| = {ref[over].abs().max().item()}")
    return err


def assert_bits_equal(got: torch.Tensor, ref: torch.Tensor, what: str) -> None:
    a = got.detach().cpu().contiguous().view(torch.int16)
    b = ref.contiguous().view(torch.int16)
    same = torch.equal(a, b)
    if not same:
        diff = (a != b).nonzero()
        raise AssertionError(f"{what}: {diff.shape[0]} differing 16-bit words, first at {diff[0].tolist()}")
    log(f"{what}: bit-identical ({a.numel()} words)")
