"""Seeded plans (who owns which physical blocks) and tensors (pool, Q, new K/V).

A plan is the state a block manager would hand to the attention step: for each
sequence, the list of physical block ids it owns in logical order, how many of
its tokens are already cached, and how many new tokens this step stores.
Lengths and block ids come from a CPU ``torch.Generator``; bulk data is drawn
as fp32 N(0, 1) from a generator on the target device and rounded to bf16
(round to nearest even, torch's conversion).

Cache rows that hold no cached token (free blocks, the unfilled tail of a
sequence's last block, and the rows the new tokens are about to be stored in)
are filled with a bf16 NaN when ``poison=True``, so any read of a row the
method must not read shows up as a non-finite output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import torch

from .configs import CONFIGS, config_seed

NAN_BF16_BITS = 0x7FC0  # quiet NaN in bfloat16


@dataclass(frozen=True)
class SeqState:
    """One sequence as the block manager sees it."""

    block_ids: Tuple[int, ...]  # physical block ids, logical order
    num_cached: int  # tokens whose K/V already sit in the cache
    num_new: int  # tokens whose K/V this step stores (1 for decode)

    @property
    def total(self) -> int:
        return self.num_cached + self.num_new


@dataclass
class Plan:
    name: str
    kind: str  # "decode" or "prefill"
    seqs: List[SeqState]
    block_size: int
    H_q: int
    H_kv: int
    d: int
    num_blocks: int
    max_blocks_per_seq: int
    layers: int = 1
    seed: int = 0

    @property
    def B(self) -> int:
        return len(self.seqs)

    @property
    def total_new(self) -> int:
        return sum(s.num_new for s in self.seqs)

    @property
    def row_elems(self) -> int:
        """Elements of one token's K (or V) row in the cache: H_kv * d."""
        return self.H_kv * self.d

    def lens(self) -> List[int]:
        return [s.total for s in self.seqs]

    def kv_tokens(self) -> int:
        """Keys read by one attention call over all sequences (decode)."""
        return sum(s.total for s in self.seqs)

    def blocks_used(self) -> int:
        return len({b for s in self.seqs for b in s.block_ids})

    def subset(self, idx: Sequence[int]) -> "Plan":
        """The same pool seen by a subset of the sequences (for sampled checks)."""
        return Plan(
            name=self.name + "[subset]", kind=self.kind,
            seqs=[self.seqs[i] for i in idx], block_size=self.block_size,
            H_q=self.H_q, H_kv=self.H_kv, d=self.d, num_blocks=self.num_blocks,
            max_blocks_per_seq=self.max_blocks_per_seq, layers=self.layers, seed=self.seed,
        )


@dataclass
class Tensors:
    """Device (or CPU) tensors of one workload.

    pool    [2, layers, num_blocks, block_size, H_kv, d] bf16; pool[0] is K, pool[1] is V
    q       [layers, T, H_q, d] bf16, T = total new tokens
    kv_new  [layers, T, 2 * H_kv * d] bf16; K of the new tokens is the first half of each
            row and V the second, so the per-layer views ``k_new``/``v_new`` have a token
            stride of 2 * H_kv * d elements (the layout of a fused projection output)
    """

    pool: torch.Tensor
    q: torch.Tensor
    kv_new: torch.Tensor
    H_kv: int
    d: int

    def k_cache(self, layer: int = 0) -> torch.Tensor:
        return self.pool[0, layer]

    def v_cache(self, layer: int = 0) -> torch.Tensor:
        return self.pool[1, layer]

    def k_new(self, layer: int = 0) -> torch.Tensor:
        T = self.kv_new.shape[1]
        D = self.H_kv * self.d
        return self.kv_new[layer, :, :D].view(T, self.H_kv, self.d)

    def v_new(self, layer: int = 0) -> torch.Tensor:
        T = self.kv_new.shape[1]
        D = self.H_kv * self.d
        return self.kv_new[layer, :, D:].view(T, self.H_kv, self.d)


def _blocks_for(tokens: int, block_size: int) -> int:
    return -(-tokens // block_size)


def _draw_lens(spec, B: int, g: torch.Generator) -> List[int]:
    if isinstance(spec, list):
        return list(spec)
    kind, lo, hi = spec
    if kind == "uniform":  # inclusive at both ends
        return [int(x) for x in torch.randint(lo, hi + 1, (B,), generator=g)]
    if kind == "loguniform":  # floor(exp(U(ln lo, ln(hi + 1))))
        u = torch.rand(B, generator=g, dtype=torch.float64)
        x = torch.exp(math.log(lo) + u * (math.log(hi + 1) - math.log(lo)))
        return [min(hi, max(lo, int(math.floor(v)))) for v in x.tolist()]
    raise ValueError(f"unknown length spec {spec!r}")


def _max_len(spec) -> int:
    if isinstance(spec, list):
        return max(spec)
    return spec[2]


def make_plan(name: str, seed: Optional[int] = None) -> Plan:
    """Seeded plan of one of the named workloads."""
    cfg = CONFIGS[name]
    seed = config_seed(name) if seed is None else seed
    g = torch.Generator().manual_seed(seed)
    bs = cfg["block_size"]
    if cfg["kind"] == "decode":
        lens = _draw_lens(cfg["lens"], cfg["B"], g)
        nblk = [_blocks_for(n, bs) for n in lens]
        num_blocks = cfg.get("num_blocks") or sum(nblk)
        perm = torch.randperm(num_blocks, generator=g).tolist()
        seqs, at = [], 0
        for n, nb in zip(lens, nblk):
            seqs.append(SeqState(tuple(perm[at:at + nb]), n - 1, 1))
            at += nb
        maxb = _blocks_for(_max_len(cfg["lens"]), bs)
    else:
        B = cfg["B"]
        lo, hi = cfg["prefix_blocks"]
        ns, nsh = cfg["shared_seqs"], cfg["shared_blocks"]
        pre = [int(x) for x in torch.randint(lo, hi + 1, (B,), generator=g)]
        pre_sh = [int(x) for x in torch.randint(nsh, hi + 1, (ns,), generator=g)]
        pre[:ns] = pre_sh
        nlo, nhi = cfg["new_tokens"]
        new = [int(x) for x in torch.randint(nlo, nhi + 1, (B,), generator=g)]
        cached = [p * bs for p in pre]
        nblk = [_blocks_for(c + n, bs) for c, n in zip(cached, new)]
        num_blocks = nsh + sum(nb - (nsh if i < ns else 0) for i, nb in enumerate(nblk))
        perm = torch.randperm(num_blocks, generator=g).tolist()
        shared = perm[:nsh]
        at = nsh
        seqs = []
        for i, (c, n, nb) in enumerate(zip(cached, new, nblk)):
            if i < ns:
                own = perm[at:at + nb - nsh]
                at += nb - nsh
                ids = tuple(shared) + tuple(own)
            else:
                ids = tuple(perm[at:at + nb])
                at += nb
            seqs.append(SeqState(ids, c, n))
        maxb = _blocks_for(hi * bs + nhi, bs)
    return Plan(
        name=name, kind=cfg["kind"], seqs=seqs, block_size=bs, H_q=cfg["H_q"],
        H_kv=cfg["H_kv"], d=cfg["d"], num_blocks=num_blocks, max_blocks_per_seq=maxb,
        layers=cfg["layers"], seed=seed,
    )


def custom_plan(
    specs: Sequence[Tuple[int, int]],
    block_size: int,
    H_q: int,
    H_kv: int,
    d: int,
    seed: int = 0,
    extra_blocks: int = 0,
    max_blocks_per_seq: Optional[int] = None,
    kind: Optional[str] = None,
    share_first: Optional[Tuple[int, int]] = None,
    layers: int = 1,
) -> Plan:
    """Plan for explicit (num_cached, num_new) pairs.

    ``share_first=(k, nb)`` makes the first k sequences use the same physical
    ids for their first nb logical blocks (their cached prefixes must cover them).
    ``extra_blocks`` free blocks are added to the pool.
    """
    g = torch.Generator().manual_seed(seed)
    nblk = [_blocks_for(c + n, block_size) for c, n in specs]
    k_sh, nb_sh = share_first if share_first else (0, 0)
    if share_first:
        for i in range(k_sh):
            assert specs[i][0] >= nb_sh * block_size, "shared blocks must be cached prefix"
    used = nb_sh + sum(nb - (nb_sh if i < k_sh else 0) for i, nb in enumerate(nblk))
    num_blocks = used + extra_blocks
    perm = torch.randperm(num_blocks, generator=g).tolist()
    shared = perm[:nb_sh]
    at = nb_sh
    seqs = []
    for i, ((c, n), nb) in enumerate(zip(specs, nblk)):
        if i < k_sh:
            ids = tuple(shared) + tuple(perm[at:at + nb - nb_sh])
            at += nb - nb_sh
        else:
            ids = tuple(perm[at:at + nb])
            at += nb
        seqs.append(SeqState(ids, c, n))
    if kind is None:
        kind = "decode" if all(n == 1 for _, n in specs) else "prefill"
    maxb = max_blocks_per_seq if max_blocks_per_seq is not None else max(nblk + [1])
    return Plan(
        name="custom", kind=kind, seqs=seqs, block_size=block_size, H_q=H_q, H_kv=H_kv,
        d=d, num_blocks=num_blocks, max_blocks_per_seq=maxb, layers=layers, seed=seed,
    )


def _history_rows(plan: Plan) -> torch.Tensor:
    """[num_blocks, block_size] bool: True where a row holds an already cached token."""
    bs = plan.block_size
    hist = torch.zeros(plan.num_blocks, bs, dtype=torch.bool)
    for s in plan.seqs:
        for j, blk in enumerate(s.block_ids):
            filled = min(max(s.num_cached - j * bs, 0), bs)
            if filled:
                hist[blk, :filled] = True
    return hist


def make_tensors(
    plan: Plan,
    device="cpu",
    poison: bool = True,
    seed: Optional[int] = None,
    layers: Optional[Sequence[int]] = None,
) -> Tensors:
    """Fill the pool and the new rows of ``plan`` with seeded bf16 N(0, 1) data.

    ``layers`` restricts which layers' pool slices get random data (the rest stay
    uninitialised memory); by default all do.
    """
    seed = plan.seed if seed is None else seed
    device = torch.device(device)
    g = torch.Generator(device=device).manual_seed(seed)
    L, NB, bs, H, d = plan.layers, plan.num_blocks, plan.block_size, plan.H_kv, plan.d
    pool = torch.empty(2, L, NB, bs, H, d, dtype=torch.bfloat16, device=device)
    fill = range(L) if layers is None else layers
    for layer in fill:
        for kv in range(2):
            pool[kv, layer].copy_(
                torch.randn(NB, bs, H, d, generator=g, device=device, dtype=torch.float32)
            )
    if poison:
        free = (~_history_rows(plan)).to(device)
        pool.view(torch.int16).masked_fill_(
            free.view(1, 1, NB, bs, 1, 1), NAN_BF16_BITS
        )
    T = plan.total_new
    q = torch.randn(L, T, plan.H_q, d, generator=g, device=device, dtype=torch.float32).to(
        torch.bfloat16
    )
    kv_new = torch.randn(L, T, 2 * H * d, generator=g, device=device, dtype=torch.float32).to(
        torch.bfloat16
    )
    return Tensors(pool=pool, q=q, kv_new=kv_new, H_kv=H, d=d)
