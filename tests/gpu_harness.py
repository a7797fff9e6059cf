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


def bf16_brackets(ref: torch.Tensor):
    """The two bf16 values that bracket each float64 reference value: the
    largest bf16 <= ref and the smallest bf16 >= ref (both equal ref when it is
    a bf16 value).  bf16 keeps 8 significant bits, so for |ref| in
    [2^(e-1), 2^e) the grid spacing is 2^(e-8) (frexp gives e exactly);
    below the smallest normal (2^-126) it is 2^-133."""
    _, e = torch.frexp(ref)
    spacing = torch.exp2((e.to(torch.float64) - 8).clamp_min(-133))
    return torch.floor(ref / spacing) * spacing, torch.ceil(ref / spacing) * spacing


def within_bar(got: torch.Tensor, ref: torch.Tensor, tol: float = TOL) -> torch.Tensor:
    """The parity bar for bf16 attention outputs, element by element: within
    ``tol`` of the float64 reference, or equal to one of the two bf16 values
    that bracket it (a faithful rounding of the exact result).  The second
    clause only matters where bf16 itself cannot meet ``tol``: from |o| = 2 up
    the bf16 spacing is 2^-6 or more, and from |o| = 4 up even the correctly
    rounded value can lie 2^-6 > 1e-2 away, so no bf16 output can be within
    ``tol`` of every real there."""
    lo, hi = bf16_brackets(ref)
    return ((got - ref).abs() <= tol) | (got == lo) | (got == hi)


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
    """Every element within the bar of ``within_bar``.  Logs the largest error,
    how many elements passed only as a bracketing bf16 value, and the largest
    error among elements with |o| >= 4 (where bf16 spacing exceeds 2 * tol)."""
    g = got.detach().float().cpu().double()
    assert g.shape == ref.shape, f"{what}: shape {tuple(g.shape)} vs oracle {tuple(ref.shape)}"
    assert torch.isfinite(g).all(), f"{what}: non-finite GPU output"
    assert torch.isfinite(ref).all(), f"{what}: non-finite oracle output"
    diff = (g - ref).abs()
    err = diff.max().item() if g.numel() else 0.0
    ok = within_bar(g, ref, tol)
    by_bracket = int((ok & (diff > tol)).sum())
    big = ref.abs() >= 4
    nbig = int(big.sum())
    err_big = diff[big].max().item() if nbig else 0.0
    log(f"{what}: max abs err {err:.3e} over {g.numel()} values; {nbig} with |o| >= 4 "
        f"(max err among them {err_big:.3e}); {by_bracket} beyond {tol:g} accepted as a "
        f"bracketing bf16 value")
    bad = ~ok
    assert not bad.any(), (f"{what}: {int(bad.sum())} values beyond the bar, worst "
                           f"{diff[bad].max().item()} at |o| = {ref[bad].abs().max().item()}")
    return err


def assert_bits_equal(got: torch.Tensor, ref: torch.Tensor, what: str) -> None:
    a = got.detach().cpu().contiguous().view(torch.int16)
    b = ref.contiguous().view(torch.int16)
    same = torch.equal(a, b)
    if not same:
        diff = (a != b).nonzero()
        raise AssertionError(f"{what}: {diff.shape[0]} differing 16-bit words, first at {diff[0].tolist()}")
    log(f"{what}: bit-identical ({a.numel()} words)")
