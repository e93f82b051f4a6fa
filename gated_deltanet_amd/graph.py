"""Pre-recorded rounds: a sequence of library calls captured once into a HIP
graph and replayed (Flide section 3.3.2: execution graphs recorded per
capacity bucket, with every round-dependent value in device buffers).

Every launch of the library takes its grid from host-known capacities
(``level_cap``, ``fork_cap``, tile and chunk capacities) and reads the round's
actual counts from the workspace, and no call issues a memset, so the
calls of one round can be captured as they are.  A graph stays valid for
any later round whose tree description, inputs and outputs live in the
same buffers with the same capacities: refill the buffers, replay.
"""
from __future__ import annotations

from typing import Callable

import torch


class StepGraph:
    """Capture ``fn`` (library calls on torch's current stream) into a graph.

    ``fn`` runs ``warmup`` times eagerly on a side stream first, so every
    one-time setup inside the library (kernel attributes, device queries)
    happens outside the capture.
    """

    def __init__(self, fn: Callable[[], None], warmup: int = 1):
        self.fn = fn
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(warmup):
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            fn()
        torch.cuda.synchronize()

    def replay(self) -> None:
        self.graph.replay()
