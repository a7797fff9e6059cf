"""Logits for the sampling measurement: one decode step of 256 sequences over
Qwen3's 151936-token vocabulary, bf16, as a model's head would hand them over.
Seeded and synthetic (scaled normal logits); no sampling arithmetic here."""
from __future__ import annotations

import torch

SAMPLE_DECODE = dict(B=256, V=151936, scale=4.0, temperature=(0.3, 1.5), seed=4001)


def make_logits(device, cfg=SAMPLE_DECODE):
    """(logits [B, V] bf16, temperatures [B] fp32, seeds [B] int64, offsets [B] int64)."""
    g = torch.Generator().manual_seed(cfg["seed"])
    lo, hi = cfg["temperature"]
    temps = lo + (hi - lo) * torch.rand(cfg["B"], generator=g)
    seeds = torch.randint(0, 2 ** 62, (cfg["B"],), generator=g, dtype=torch.int64)
    offsets = torch.randint(0, 4096, (cfg["B"],), generator=g, dtype=torch.int64)
    dg = torch.Generator(device=device).manual_seed(cfg["seed"] + 1)
    logits = (torch.randn(cfg["B"], cfg["V"], generator=dg, device=device) * cfg["scale"]).to(torch.bfloat16)
    return logits, temps.to(device), seeds.to(device), offsets.to(device)
