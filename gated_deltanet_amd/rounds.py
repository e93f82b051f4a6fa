"""Host-side planning of a round: page tables and launch capacities.

The caller builds its round's tree on the host (it knows its requests), so
the host also sizes the fixed capacities the launches use (Flide section
3.3.2: captured shapes carry fixed capacities for segments and chunks) and
assigns K/V pages: every live segment gets fresh pages, while a cached
segment keeps the pages its earlier pass wrote (ForkServe item 1: a child
aliases its ancestors' pages).  Per-token work happens only on the device.

A round may also be planned into a capacity bucket -- a stream capacity T, a
segment capacity S, and level / fork-point / depth capacities -- larger than
itself: the stream is padded at its tail (FK_PAD_TOKEN) and the unused
segment slots are marked (FK_UNUSED_SEGMENT), so a graph captured once for
the bucket replays any round that fits (Flide section 3.3.2).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional, Sequence

import numpy as np

from ._lib import FK_MAX_DEPTH, FK_TILE_TOKENS
from .api import TreeMeta, make_tree_meta

PAGE = FK_TILE_TOKENS
PAD_TOKEN = -1        # FK_PAD_TOKEN
UNUSED_SEGMENT = -1   # FK_UNUSED_SEGMENT


@dataclass(frozen=True)
class Bucket:
    """Capacities of a family member: stream tokens, segment slots, tree
    levels, live segments per level, distinct fork points."""
    T: int
    S: int
    max_depth: int
    level_cap: int
    fork_cap: int


@dataclass
class RoundPlan:
    meta: TreeMeta
    seg_len: np.ndarray        # host copy of segment lengths (the round's own segments)
    seg_page_off: np.ndarray   # host copy of the page CSR (capacity-padded)
    seg_pages: np.ndarray
    n_pages: int
    pages_used: int            # pages this round's live segments occupy (from first_page)
    bucket: Optional[Bucket] = None
    arrays: Optional[Dict[str, np.ndarray]] = None   # the padded host arrays behind meta


def seg_lengths(tok_seg, seg_cached_len) -> np.ndarray:
    S = len(seg_cached_len)
    ts = np.asarray(tok_seg, np.int64)
    live = np.bincount(ts[ts >= 0], minlength=S)[:S]
    cl = np.asarray(seg_cached_len, np.int64)
    return np.where(cl > 0, cl, live).astype(np.int64)


def capacities(seg_parent, seg_fork, seg_cached_len):
    """(max_depth, level_cap, fork_cap) that exactly fit the round."""
    par = np.asarray(seg_parent)
    fk = np.asarray(seg_fork)
    cl = np.asarray(seg_cached_len)
    S = len(par)
    depth = np.zeros(S, np.int64)
    for s in range(S):
        d, i = 0, s
        while par[i] >= 0:
            i = par[i]
            d += 1
            if d > S:
                raise ValueError("cycle in seg_parent")
        depth[s] = d
    live = cl == 0
    per_level = np.bincount(depth[live], minlength=1)
    forks = set()
    for c in range(S):
        p = par[c]
        if live[c] and p >= 0 and live[p]:
            forks.add((int(p), int(fk[c])))
    return int(depth.max()) + 1, int(max(per_level.max(), 1)), len(forks)


def _ladder(n: int, floor: int, steps: int) -> int:
    """Smallest value >= n on a geometric ladder with ``steps`` rungs per
    doubling, starting at ``floor``."""
    c = floor
    while True:
        for k in range(steps):
            v = c + c * k // steps
            if v >= n:
                return v
        c *= 2


def bucket_for(T: int, S: int, max_depth: int, level_cap: int, fork_cap: int) -> Bucket:
    """The smallest member of the capacity family that holds a round: the
    stream on quarter steps of a doubling ladder (at least 1,024 tokens), the
    segment slots, level and fork-point capacities on half steps (at least
    16), the depth as 2, 4 or 8 levels."""
    s_cap = _ladder(S, 16, 2)
    depth = 2 if max_depth <= 2 else 4 if max_depth <= 4 else FK_MAX_DEPTH
    return Bucket(T=_ladder(T, 1024, 4), S=s_cap, max_depth=depth, level_cap=min(_ladder(level_cap, 16, 2), s_cap),
                  fork_cap=_ladder(max(fork_cap, 1), 16, 2))


def plan_arrays(tok_seg, seg_parent, seg_fork, seg_cached_len,
                cached_pages: Optional[Dict[int, Sequence[int]]] = None, first_page: int = 0,
                seg_state_in=None, seg_state_out=None, bucket: Optional[Bucket] = None):
    """Host arrays of a round (pages assigned), padded into ``bucket`` when
    one is given.  Returns (arrays, lengths, pages used, exact capacities)."""
    lens = seg_lengths(tok_seg, seg_cached_len)
    cl = np.asarray(seg_cached_len, np.int64)
    S, T = len(lens), len(tok_seg)
    counts = np.zeros(S, np.int64)
    lists = []
    nxt = first_page
    for s in range(S):
        need = -(-int(lens[s]) // PAGE)
        if cl[s] > 0:
            pg = np.asarray((cached_pages or {}).get(s, []), np.int64)
        else:
            pg = np.arange(nxt, nxt + need, dtype=np.int64)
            nxt += need
        lists.append(pg)
        counts[s] = len(pg)
    caps = capacities(seg_parent, seg_fork, seg_cached_len)
    Tc, Sc = (bucket.T, bucket.S) if bucket else (T, S)
    if bucket and (T > bucket.T or S > bucket.S or caps[0] > bucket.max_depth or caps[1] > bucket.level_cap
                   or caps[2] > bucket.fork_cap):
        raise ValueError(f"round (T={T}, S={S}, caps={caps}) does not fit {bucket}")
    off = np.zeros(Sc + 1, np.int64)
    off[1:S + 1] = np.cumsum(counts)
    off[S + 1:] = off[S]
    pages = np.concatenate(lists) if lists else np.zeros(0, np.int64)

    def pad(a, n, fill):
        out = np.full(n, fill, np.int32)
        a = np.asarray(a, np.int64)
        out[:len(a)] = a
        return out

    arrays = {
        "tok_seg": pad(tok_seg, Tc, PAD_TOKEN),
        "seg_parent": pad(seg_parent, Sc, -1),
        "seg_fork": pad(seg_fork, Sc, 0),
        "seg_cached_len": pad(seg_cached_len, Sc, UNUSED_SEGMENT),
        "seg_page_off": off.astype(np.int32),
        "seg_pages": pages.astype(np.int32),
        "seg_state_in": pad(seg_state_in if seg_state_in is not None else np.full(S, -1), Sc, -1),
        "seg_state_out": pad(seg_state_out if seg_state_out is not None else np.full(S, -1), Sc, -1),
    }
    return arrays, lens, nxt - first_page, caps


def plan_round(tok_seg, seg_parent, seg_fork, seg_cached_len,
               cached_pages: Optional[Dict[int, Sequence[int]]] = None, first_page: int = 0,
               n_pages: Optional[int] = None, seg_state_in=None, seg_state_out=None,
               n_state_in: int = 0, n_state_out: int = 0, bucket: Optional[Bucket] = None,
               device="cuda") -> RoundPlan:
    """Assign pages and capacities and upload the tree description.

    Live segments get consecutive fresh pages starting at ``first_page``;
    cached segment s uses ``cached_pages[s]``.  ``n_pages`` is the pool size
    (default: just enough for this round).  With ``bucket`` the round is
    padded into that bucket's capacities (tail padding, unused segment slots).
    """
    arrays, lens, used, caps = plan_arrays(tok_seg, seg_parent, seg_fork, seg_cached_len, cached_pages,
                                           first_page, seg_state_in, seg_state_out, bucket)
    pages = arrays["seg_pages"]
    if n_pages is None:
        n_pages = max(first_page + used, int(pages.max()) + 1 if pages.size else 1)
    max_depth, level_cap, fork_cap = caps
    if bucket:
        max_depth, level_cap, fork_cap = bucket.max_depth, bucket.level_cap, bucket.fork_cap
    a = arrays
    meta = make_tree_meta(a["tok_seg"], a["seg_parent"], a["seg_fork"], a["seg_cached_len"], a["seg_page_off"],
                          a["seg_pages"], n_pages, a["seg_state_in"], a["seg_state_out"], n_state_in, n_state_out,
                          max_depth, level_cap, max(fork_cap, 1), device=device)
    return RoundPlan(meta=meta, seg_len=lens, seg_page_off=a["seg_page_off"], seg_pages=pages, n_pages=n_pages,
                     pages_used=used, bucket=bucket, arrays=arrays)
