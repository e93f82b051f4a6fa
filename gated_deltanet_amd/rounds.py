"""Host-side planning of a round: page tables and launch capacities.

The caller builds its round's tree on the host (it knows its requests), so
the host also sizes the fixed capacities the launches use (Flide section
3.3.2: captured shapes carry fixed capacities for segments and chunks) and
assigns K/V pages: every live segment gets fresh pages, while a cached
segment keeps the pages its earlier pass wrote (ForkServe item 1: a child
aliases its ancestors' pages).  Per-token work happens only on the device.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional, Sequence

import numpy as np

from ._lib import FK_TILE_TOKENS
from .api import TreeMeta, make_tree_meta

PAGE = FK_TILE_TOKENS


@dataclass
class RoundPlan:
    meta: TreeMeta
    seg_len: np.ndarray        # host copy of segment lengths
    seg_page_off: np.ndarray   # host copy of the page CSR
    seg_pages: np.ndarray
    n_pages: int
    pages_used: int            # pages this round's live segments occupy (from first_page)


def seg_lengths(tok_seg, seg_cached_len) -> np.ndarray:
    S = len(seg_cached_len)
    live = np.bincount(np.asarray(tok_seg, np.int64), minlength=S)[:S]
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


def plan_round(tok_seg, seg_parent, seg_fork, seg_cached_len,
               cached_pages: Optional[Dict[int, Sequence[int]]] = None, first_page: int = 0,
               n_pages: Optional[int] = None, seg_state_in=None, seg_state_out=None,
               n_state_in: int = 0, n_state_out: int = 0, device="cuda") -> RoundPlan:
    """Assign pages and capacities and upload the tree description.

    Live segments get consecutive fresh pages starting at ``first_page``;
    cached segment s uses ``cached_pages[s]``.  ``n_pages`` is the pool size
    (default: just enough for this round).
    """
    lens = seg_lengths(tok_seg, seg_cached_len)
    cl = np.asarray(seg_cached_len)
    S = len(lens)
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
    off = np.zeros(S + 1, np.int64)
    off[1:] = np.cumsum(counts)
    pages = np.concatenate(lists) if lists else np.zeros(0, np.int64)
    max_depth, level_cap, fork_cap = capacities(seg_parent, seg_fork, seg_cached_len)
    if n_pages is None:
        n_pages = max(nxt, int(pages.max()) + 1 if pages.size else 1)
    meta = make_tree_meta(tok_seg, seg_parent, seg_fork, seg_cached_len, off, pages, n_pages,
                          seg_state_in, seg_state_out, n_state_in, n_state_out, max_depth,
                          level_cap, max(fork_cap, 1), device=device)
    return RoundPlan(meta=meta, seg_len=lens, seg_page_off=off, seg_pages=pages, n_pages=n_pages,
                     pages_used=nxt - first_page)
