"""Packed (non-paged) varlen prefill workload: the no-prefix form of the
devpress page's varlen call, q/k/v as row views of one fused projection
buffer per token.  Seeded and synthetic; no attention arithmetic here."""
from __future__ import annotations

from typing import List, Tuple

import torch

PACKED_PREFILL = dict(B=16, new_tokens=(128, 2048), H_q=16, H_kv=8, d=128, seed=2001)


def packed_lens(cfg=PACKED_PREFILL) -> List[int]:
    g = torch.Generator().manual_seed(cfg["seed"])
    lo, hi = cfg["new_tokens"]
    return [int(x) for x in torch.randint(lo, hi + 1, (cfg["B"],), generator=g)]


def make_packed(device, cfg=PACKED_PREFILL) -> Tuple[List[int], torch.Tensor, torch.Tensor]:
    """Returns (lengths, cu_seqlens [B+1] int32 on device, fused [T, (H_q+2H_kv)*d] bf16)."""
    lens = packed_lens(cfg)
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    width = (cfg["H_q"] + 2 * cfg["H_kv"]) * cfg["d"]
    gen = torch.Generator(device=device).manual_seed(cfg["seed"] + 1)
    fused = torch.randn(cu[-1], width, generator=gen, device=device, dtype=torch.float32)
    fused = fused.to(torch.bfloat16)
    return lens, torch.tensor(cu, dtype=torch.int32, device=device), fused


def split_fused(fused: torch.Tensor, cfg=PACKED_PREFILL):
    """q [T, H_q, d], k/v [T, H_kv, d] as row-strided views of the fused buffer."""
    H_q, H_kv, d = cfg["H_q"], cfg["H_kv"], cfg["d"]
    q = fused[:, : H_q * d].view(-1, H_q, d)
    k = fused[:, H_q * d: (H_q + H_kv) * d].view(-1, H_kv, d)
    v = fused[:, (H_q + H_kv) * d:].view(-1, H_kv, d)
    return q, k, v
