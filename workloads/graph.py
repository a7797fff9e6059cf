"""Decode step for the graph-capture measurement: 28 layers of Qwen3-0.6B
attention shapes at small batches, where launch overhead is a large part of
the step.  Seeded and synthetic; no attention arithmetic here."""
from __future__ import annotations

import torch

from .gen import Plan, custom_plan

GRAPH_DECODE = dict(layers=28, H_q=16, H_kv=8, d=128, block_size=256, max_batch=64,
                    context=(128, 2048), batches=(1, 5, 16, 64), seed=3001)


def graph_plan(cfg=GRAPH_DECODE) -> Plan:
    """max_batch decode sequences with context lengths U[context] (inclusive);
    a step of batch b runs the first b of them."""
    g = torch.Generator().manual_seed(cfg["seed"])
    lo, hi = cfg["context"]
    lens = [int(x) for x in torch.randint(lo, hi + 1, (cfg["max_batch"],), generator=g)]
    return custom_plan([(n - 1, 1) for n in lens], cfg["block_size"], cfg["H_q"], cfg["H_kv"],
                       cfg["d"], seed=cfg["seed"], layers=cfg["layers"])
