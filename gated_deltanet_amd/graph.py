"""Pre-recorded rounds (Flide section 3.3.2: execution graphs recorded once
per capacity bucket, every round-dependent value in device buffers, padding
only at the tail).

Every launch of the library takes its grid from host-known capacities (the
tree description's T and S, ``level_cap``, ``fork_cap``, ``max_depth``) and
reads the round's actual counts from the workspace, and no call issues a
memset, so the calls of one round can be captured as they are.  A graph
captured for a bucket replays any later round that fits the bucket once its
tree description and inputs are refilled in place (``BucketRound.load``):
padding tokens and unused segment slots get no work, and every output row
of the round has the bits an exact-size run gives.
"""
from __future__ import annotations

from typing import Callable, Dict

import numpy as np
import torch

from .api import TreeMeta
from .rounds import Bucket


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


class BucketRound:
    """The tree description of a capacity bucket in fixed device buffers:
    ``meta`` carries the bucket's capacities and stays valid (same pointers)
    for every round loaded into it, so a graph captured over it replays any
    round that fits.  ``page_cap``: page-list entries (the round's own pages
    plus the pages of its cached histories); ``n_pages``, ``n_state_in``,
    ``n_state_out``: the caller's pool and state-slot sizes."""

    FIELDS = ("tok_seg", "seg_parent", "seg_fork", "seg_cached_len", "seg_page_off", "seg_pages",
              "seg_state_in", "seg_state_out")

    def __init__(self, bucket: Bucket, page_cap: int, n_pages: int, n_state_in: int = 0, n_state_out: int = 0,
                 device="cuda"):
        self.bucket = bucket
        sizes = {"tok_seg": max(bucket.T, 1), "seg_page_off": bucket.S + 1, "seg_pages": max(page_cap, 1)}
        self.buf = {f: torch.zeros(sizes.get(f, bucket.S), dtype=torch.int32, device=device) for f in self.FIELDS}
        self.meta = TreeMeta(T=bucket.T, S=bucket.S, max_depth=bucket.max_depth, level_cap=bucket.level_cap,
                             fork_cap=bucket.fork_cap, n_pages=n_pages, n_state_in=n_state_in,
                             n_state_out=n_state_out, **self.buf)

    def load(self, arrays: Dict[str, np.ndarray]) -> None:
        """Copy a round's padded host arrays (``rounds.plan_arrays`` with this
        bucket) into the fixed buffers, in place, on torch's current stream."""
        for f in self.FIELDS:
            a = np.ascontiguousarray(arrays[f], np.int32)
            dst = self.buf[f]
            if f == "seg_pages":
                assert a.size <= dst.numel(), "page list exceeds the bucket's page capacity"
            else:
                assert a.size == dst.numel(), (f, a.size, dst.numel())
            if a.size:
                dst[:a.size].copy_(torch.from_numpy(a), non_blocking=False)


class GraphFamily:
    """Step graphs indexed by capacity bucket (Flide section 3.3.2).
    ``factory(bucket)`` returns an object whose ``step()`` issues one round's
    library calls on buffers sized for the bucket; its graph is captured on
    the bucket's first use and replayed for every later round there."""

    def __init__(self, factory: Callable[[Bucket], object]):
        self.factory = factory
        self.members: Dict[Bucket, tuple] = {}

    def member(self, bucket: Bucket):
        """(the bucket's object, its captured graph or None before capture)."""
        if bucket not in self.members:
            self.members[bucket] = (self.factory(bucket), None)
        return self.members[bucket]

    def replay(self, bucket: Bucket) -> object:
        """Replay the bucket's graph (captured now if this is its first use);
        the caller has loaded the round into the bucket's object."""
        obj, graph = self.member(bucket)
        if graph is None:
            graph = StepGraph(obj.step)
            self.members[bucket] = (obj, graph)
        graph.replay()
        return obj
