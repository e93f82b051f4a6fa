"""Seeded synthetic tensors drawn directly on the GPU (torch), for workloads
too large to draw on the host (the resume workload carries 64 x 16,384
history tokens).  Same recipe as ``tensors``: q/k/v ~ N(0,1), GDN q and k
L2-normalised per head, a = sigmoid(N(mu_a, 1)), b = sigmoid(N(0, 1)),
activations rounded to bf16; only the random stream differs (torch's
generator instead of PCG64), so these values are for timing runs and for
requests that no oracle comparison reads.
"""
from __future__ import annotations

from typing import Dict

import torch

from .tensors import NAMES, Shapes


def draw_stream(T: int, sh: Shapes, seed: int, mu_a: float, device="cuda",
                names=NAMES, chunk: int = 1 << 17) -> Dict[str, torch.Tensor]:
    """Stream-order tensors of T tokens (bf16 activations, fp32 gates)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = {}
    for name in names:
        dims = sh.dims(name)
        dt = torch.float32 if name in ("ga", "gb") else torch.bfloat16
        x = torch.empty((T,) + dims, dtype=dt, device=device)
        for t0 in range(0, T, chunk):
            n = min(chunk, T - t0)
            z = torch.randn((n,) + dims, generator=gen, device=device, dtype=torch.float32)
            if name in ("gq", "gk"):
                z = z / z.norm(dim=-1, keepdim=True)
            elif name == "ga":
                z = torch.sigmoid(z + mu_a)
            elif name == "gb":
                z = torch.sigmoid(z)
            x[t0:t0 + n] = z.to(dt)
        out[name] = x
    return out
