"""Seeded tensors for every segment of a round.

Every segment draws from its own substream, derived from
``SeedSequence(seed)`` -> request -> segment creation index, so a branch has
the same values whether it runs alone or inside any mixture.  Per segment the
draw order is: attention q, k, v; GDN q, k, v; a_pre, b_pre, each a
standard-normal array drawn as float32 from PCG64.

Value recipe (the workload statement): q/k/v ~ N(0,1); GDN q and k
L2-normalised per head (in fp64, before rounding); a = sigmoid(N(mu_a, 1)),
b = sigmoid(N(0, 1)), stored as fp32.  Activations are then rounded to the
workload dtype (bf16 round-to-nearest-even, or fp32).  The rounded values are
the ground truth for both sides; ``Inputs.f64(name)`` widens them exactly.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, List, Optional

import numpy as np

from .trees import Tree

ACT = ("aq", "ak", "av", "gq", "gk", "gv")   # activations (workload dtype)
GATE = ("ga", "gb")                          # decay / write strength (fp32)
NAMES = ACT + GATE


def to_f32(x: np.ndarray) -> np.ndarray:
    """Round to fp32 (RNE)."""
    return np.asarray(x).astype(np.float32)


def to_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bf16 (RNE via fp32); returns the uint16 bit patterns."""
    x32 = np.ascontiguousarray(np.asarray(x).astype(np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclass(frozen=True)
class Shapes:
    Hq: int
    Hkv: int
    d: int
    Hk: int
    Hv: int
    dk: int
    dv: int

    def dims(self, name: str):
        return {"aq": (self.Hq, self.d), "ak": (self.Hkv, self.d), "av": (self.Hkv, self.d),
                "gq": (self.Hk, self.dk), "gk": (self.Hk, self.dk), "gv": (self.Hv, self.dv),
                "ga": (self.Hv,), "gb": (self.Hv,)}[name]


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _l2n(x):
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


class SeedTree:
    """SeedSequence(seed) -> child per request stream -> child per segment key.

    ``spawn_key=(r, key)`` is exactly ``SeedSequence(seed).spawn(..)[r].spawn(..)[key]``,
    without the statefulness of ``spawn``.
    """

    def __init__(self, seed: int):
        self.seed = int(seed)

    def generator(self, request_stream: int, key: int) -> np.random.Generator:
        ss = np.random.SeedSequence(self.seed, spawn_key=(int(request_stream), int(key)))
        return np.random.Generator(np.random.PCG64(ss))


def draw_segment(seeds: SeedTree, request_stream: int, key: int, n: int, sh: Shapes,
                 mu_a: float, dtype: str) -> Dict[str, np.ndarray]:
    """Raw (stored) tensors of one segment: uint16 bf16 bits or float32."""
    gen = seeds.generator(request_stream, key)
    rnd = to_bf16 if dtype == "bf16" else to_f32
    out = {}
    for name in NAMES:
        z = gen.standard_normal((n,) + sh.dims(name), dtype=np.float32)
        if name in ("gq", "gk"):
            out[name] = rnd(_l2n(z.astype(np.float64)))
        elif name == "ga":
            out[name] = to_f32(_sigmoid(z.astype(np.float64) + mu_a))
        elif name == "gb":
            out[name] = to_f32(_sigmoid(z.astype(np.float64)))
        else:
            out[name] = rnd(z)
    return out


@dataclass
class Inputs:
    """Stream-order tensors plus cached-history tensors (raw storage).

    Cached segments contribute rows to ``hist`` (in segment-index order)
    instead of the stream; ``hist_off[s]`` is segment s's first history row.
    """
    dtype: str
    shapes: Shapes
    tree: Tree
    raw: Dict[str, np.ndarray]
    hist: Dict[str, np.ndarray]
    hist_off: np.ndarray

    def f64(self, name: str, hist: bool = False) -> np.ndarray:
        x = (self.hist if hist else self.raw)[name]
        if x.dtype == np.uint16:
            return bf16_to_f64(x)
        return x.astype(np.float64)


def draw_inputs(tree: Tree, shapes: Shapes, seed: int, dtype: str = "bf16",
                mu_a: float = 3.0, request_streams: Optional[List[int]] = None,
                cache: Optional[dict] = None) -> Inputs:
    """Draw every segment's tensors and lay them out in stream order.

    ``request_streams[r]`` names the seed stream that request ``r`` of this
    tree uses (for a branch run alone: its request's index in the full round).
    ``cache`` (optional dict) keeps each segment's draw for later calls with
    the same seed, shapes and dtype (several paths of one request share their
    ancestors' values).
    """
    assert tree.tok_seg is not None, "flatten() the tree first"
    assert dtype in ("bf16", "f32")
    seeds = SeedTree(seed)
    vals = []
    for s in tree.segs:
        r = request_streams[s.request] if request_streams is not None else s.request
        key = (seed, shapes, dtype, mu_a, r, s.key, s.length)
        if cache is not None and key in cache:
            vals.append(cache[key])
            continue
        vals.append(draw_segment(seeds, r, s.key, s.length, shapes, mu_a, dtype))
        if cache is not None:
            cache[key] = vals[-1]
    raw, hist = {}, {}
    cached_ids = [i for i, s in enumerate(tree.segs) if s.cached]
    hist_off = np.zeros(tree.S + 1, np.int64)
    acc = 0
    for i in range(tree.S):
        hist_off[i] = acc
        if tree.segs[i].cached:
            acc += tree.segs[i].length
    hist_off[tree.S] = acc
    for name in NAMES:
        empty = np.zeros((0,) + shapes.dims(name),
                         np.uint16 if (dtype == "bf16" and name in ACT) else np.float32)
        live = [vals[i][name] for i in tree.order]
        raw[name] = np.concatenate(live, 0) if live else empty
        hx = [vals[i][name] for i in cached_ids]
        hist[name] = np.concatenate(hx, 0) if hx else empty
    return Inputs(dtype=dtype, shapes=shapes, tree=tree, raw=raw, hist=hist, hist_off=hist_off)


@dataclass
class ConvInputs:
    """Inputs of the short causal convolution in front of the GDN rule.

    ``x`` [T, C] stream rows and ``hx`` [Nh, C] cached-history rows (raw
    storage, laid out like ``Inputs``), ``w`` [C, W] fp32 weights.
    """
    dtype: str
    C: int
    W: int
    x: np.ndarray
    hx: np.ndarray
    hist_off: np.ndarray
    w: np.ndarray

    def f64(self, hist: bool = False) -> np.ndarray:
        a = self.hx if hist else self.x
        return bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def draw_conv(tree: Tree, C: int, W: int, seed: int, dtype: str = "bf16",
              request_streams: Optional[List[int]] = None) -> ConvInputs:
    """Conv inputs of every segment, x ~ N(0, 1), and weights w ~ U(-1/sqrt(W),
    1/sqrt(W)) (a depthwise convolution's usual initialisation, fan-in W), so
    outputs stay within the range where a bf16 output's rounding error is
    below the bf16 bar.

    Each segment draws from ``SeedSequence(seed, spawn_key=(request, key, 1))``
    -- a stream of its own, so the tensors of ``draw_inputs`` are unchanged
    and a branch again gets the same values alone or in any mixture.  The
    weights come from ``spawn_key=(2**30 + 1,)``.
    """
    assert tree.tok_seg is not None, "flatten() the tree first"
    assert dtype in ("bf16", "f32")
    rnd = to_bf16 if dtype == "bf16" else to_f32
    vals = []
    for s in tree.segs:
        r = request_streams[s.request] if request_streams is not None else s.request
        ss = np.random.SeedSequence(int(seed), spawn_key=(int(r), int(s.key), 1))
        gen = np.random.Generator(np.random.PCG64(ss))
        vals.append(rnd(gen.standard_normal((s.length, C), dtype=np.float32)))
    wgen = np.random.Generator(np.random.PCG64(np.random.SeedSequence(int(seed), spawn_key=(2**30 + 1,))))
    w = to_f32(wgen.uniform(-1.0, 1.0, (C, W)) / np.sqrt(W))
    store = np.uint16 if dtype == "bf16" else np.float32
    live = [vals[i] for i in tree.order]
    cached_ids = [i for i, s in enumerate(tree.segs) if s.cached]
    hist_off = np.zeros(tree.S + 1, np.int64)
    acc = 0
    for i in range(tree.S):
        hist_off[i] = acc
        if tree.segs[i].cached:
            acc += tree.segs[i].length
    hist_off[tree.S] = acc
    x = np.concatenate(live, 0) if live else np.zeros((0, C), store)
    hx = np.concatenate([vals[i] for i in cached_ids], 0) if cached_ids else np.zeros((0, C), store)
    return ConvInputs(dtype=dtype, C=C, W=W, x=x, hx=hx, hist_off=hist_off, w=w)
