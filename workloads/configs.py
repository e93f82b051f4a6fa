"""The five decision-request workloads (tree recipe, shapes, dtype, seed).

Config i uses seed ``1000 + i``; the tree structure draws from its own
substream (request stream ``-1`` is not used: structure uses
``SeedSequence(seed, spawn_key=(1 << 30,))``) so structure and tensors are
independent.

0  tiny: 1 request, trunk 48, branches 6/8/10; fp32; attention 4q/1kv d64;
   GDN 2 heads dk=dv=32.
1  mixture: 16 requests, trunk ~U[512,2048], 4-8 branches of U[16,48]; bf16;
   attention 16q/2kv d128; GDN 16/16 heads, 128/128.
2  agent fan-out: 10 sessions, trunk 4096 -> 4 x 256 -> each 4 x 32 (pages of
   16, all page-aligned); attention 32q/4kv; GDN 16 k / 32 v heads.
3  long shared context: 4 requests, trunk 32768, 16 branches of 64;
   a = sigmoid(N(4,1)); attention 32/4; GDN 16/32.
4  resume + heterogeneous trees: 64 requests, each a cached 16384-token
   history (checkpointed GDN state + paged K/V) -> 1024 new tokens -> 6
   branches of 32; random depth D ~ U{1,2,3}; every node at depth 1..D-1
   forks U{2..8} children of 32 tokens.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .tensors import Shapes
from .trees import Tree, build_tree


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    seed: int
    dtype: str
    shapes: Shapes
    mu_a: float
    page_size: int = 16


WORKLOADS = {
    0: Config(0, "tiny decision request", 1000, "f32", Shapes(4, 1, 64, 2, 2, 32, 32), 3.0),
    1: Config(1, "decision-request mixture", 1001, "bf16", Shapes(16, 2, 128, 16, 16, 128, 128), 3.0),
    2: Config(2, "agent fan-out depth 3", 1002, "bf16", Shapes(32, 4, 128, 16, 32, 128, 128), 3.0),
    3: Config(3, "long shared context", 1003, "bf16", Shapes(32, 4, 128, 16, 32, 128, 128), 4.0),
    4: Config(4, "expanding-history resume", 1004, "bf16", Shapes(32, 4, 128, 16, 32, 128, 128), 3.0),
}


def _structure_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(1 << 30,))))


def config_requests(i: int, n_requests: Optional[int] = None):
    """Per-request node lists ``(parent_local, fork, length[, cached])``."""
    cfg = WORKLOADS[i]
    rng = _structure_rng(cfg.seed)
    reqs = []
    if i == 0:
        reqs.append([(-1, 0, 48), (0, None, 6), (0, None, 8), (0, None, 10)])
    elif i == 1:
        for _ in range(16):
            trunk = int(rng.integers(512, 2049))
            nb = int(rng.integers(4, 9))
            nodes = [(-1, 0, trunk)]
            for _ in range(nb):
                nodes.append((0, None, int(rng.integers(16, 49))))
            reqs.append(nodes)
    elif i == 2:
        for _ in range(10):
            nodes = [(-1, 0, 4096)]
            for _ in range(4):
                nodes.append((0, None, 256))
                p = len(nodes) - 1
                for _ in range(4):
                    nodes.append((p, None, 32))
            reqs.append(nodes)
    elif i == 3:
        for _ in range(4):
            reqs.append([(-1, 0, 32768)] + [(0, None, 64)] * 16)
    elif i == 4:
        for _ in range(64):
            depth = int(rng.integers(1, 4))
            nodes = [(-1, 0, 16384, True), (0, None, 1024)]
            level = []
            for _ in range(6):
                nodes.append((1, None, 32))
                level.append(len(nodes) - 1)
            for _ in range(1, depth):
                nxt = []
                for p in level:
                    for _ in range(int(rng.integers(2, 9))):
                        nodes.append((p, None, 32))
                        nxt.append(len(nodes) - 1)
                level = nxt
            reqs.append(nodes)
    else:
        raise KeyError(i)
    if n_requests is not None:
        reqs = reqs[:n_requests]
    return reqs


def make_config(i: int, n_requests: Optional[int] = None) -> tuple[Config, Tree]:
    """The config's round as a flattened tree (Eq. 2 level order)."""
    tree = build_tree(config_requests(i, n_requests)).flatten()
    return WORKLOADS[i], tree
