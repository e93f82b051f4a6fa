"""Decision-request trees and their flattened stream layout.

A round is a list of requests.  Each request is a tree of segments: a trunk
(the shared state), question branches that fork from it, and possibly deeper
forks (Flide, section 3.1 and Fig. 2a; ForkServe's context tree, item 1).
A *cached* segment is a history whose keys/values and final recurrent state
were saved by an earlier pass (Flide, section 3.4); it has no tokens in the
stream.

The stream follows Flide's Eq. 2: all level-0 (trunk) segments of every
request first, then the level-1 segments, and so on, without padding.
Segments may also be laid out in any other order (Flide, section 3.2.3: the
result holds under any flat layout), which ``Tree.flatten(order=...)``
supports.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np


@dataclass
class Seg:
    request: int          # request index within the round
    key: int              # creation index within its request (seeds its tensors)
    parent: int           # global segment index of the parent, -1 for a root
    fork: int             # how many of the parent's tokens this segment sees
    length: int           # tokens (stream tokens if live, history tokens if cached)
    cached: bool = False  # history segment: K/V in saved pages, state in a slot


@dataclass
class Tree:
    segs: List[Seg]
    n_requests: int
    # stream layout, filled by flatten()
    order: List[int] = field(default_factory=list)   # segment ids in stream order
    tok_seg: Optional[np.ndarray] = None              # [T] int32

    @property
    def S(self) -> int:
        return len(self.segs)

    @property
    def T(self) -> int:
        return int(sum(s.length for s in self.segs if not s.cached))

    def depth_of(self, i: int) -> int:
        d = 0
        while self.segs[i].parent >= 0:
            i = self.segs[i].parent
            d += 1
        return d

    def flatten(self, order: Optional[Sequence[int]] = None) -> "Tree":
        """Lay live segments out in the stream (default: Eq. 2 level order)."""
        if order is None:
            depth = [self.depth_of(i) for i in range(self.S)]
            order = sorted((i for i in range(self.S) if not self.segs[i].cached),
                           key=lambda i: (depth[i], self.segs[i].request, self.segs[i].key))
        order = [int(i) for i in order]
        live = sorted(i for i in range(self.S) if not self.segs[i].cached)
        assert sorted(order) == live, "order must list every live segment once"
        self.order = order
        self.tok_seg = np.concatenate(
            [np.full(self.segs[i].length, i, np.int32) for i in order]
        ) if order else np.zeros(0, np.int32)
        return self

    def arrays(self):
        """tree_meta arrays as host numpy int32 (tok_seg, parent, fork, cached_len)."""
        assert self.tok_seg is not None, "flatten() first"
        parent = np.array([s.parent for s in self.segs], np.int32)
        fork = np.array([s.fork for s in self.segs], np.int32)
        cached = np.array([s.length if s.cached else 0 for s in self.segs], np.int32)
        return self.tok_seg, parent, fork, cached

    def children(self, i: int) -> List[int]:
        return [j for j, s in enumerate(self.segs) if s.parent == i]

    def leaves(self) -> List[int]:
        has_child = set(s.parent for s in self.segs if s.parent >= 0)
        return [i for i, s in enumerate(self.segs) if not s.cached and i not in has_child]

    def branch_tokens(self) -> int:
        """Tokens of live segments below a root (the branch-token count)."""
        return int(sum(s.length for s in self.segs if not s.cached and s.parent >= 0
                       and not self.segs[s.parent].cached))

    def root_live_tokens(self) -> int:
        return self.T - self.branch_tokens()


def build_tree(requests: Sequence[Sequence[tuple]]) -> Tree:
    """Build a round from per-request node lists.

    Each request is a list of tuples ``(parent_local, fork, length[, cached])``
    in creation order; ``parent_local`` indexes the same list (-1 = root) and
    must refer to an earlier node.  ``fork=None`` means "at the parent's end".
    """
    segs: List[Seg] = []
    for r, nodes in enumerate(requests):
        base = len(segs)
        for key, node in enumerate(nodes):
            p, f, n = node[0], node[1], node[2]
            cached = bool(node[3]) if len(node) > 3 else False
            if p >= 0:
                assert p < key, "parents precede children"
                if f is None:
                    f = segs[base + p].length
                gp = base + p
            else:
                f = 0 if f is None else f
                gp = -1
            segs.append(Seg(request=r, key=key, parent=gp, fork=int(f),
                            length=int(n), cached=cached))
    return Tree(segs=segs, n_requests=len(requests))


def subtree_path(tree: Tree, leaf: int) -> tuple[Tree, List[int]]:
    """The root-to-``leaf`` chain of ``tree`` as its own round ("asked alone").

    Segments keep their request/key identity (so their tensors are the same)
    and their boundaries.  Returns the new tree and the map new->old index.
    """
    chain = []
    i = leaf
    while i >= 0:
        chain.append(i)
        i = tree.segs[i].parent
    chain.reverse()
    remap = {old: new for new, old in enumerate(chain)}
    segs = []
    for old in chain:
        s = tree.segs[old]
        segs.append(Seg(request=0, key=s.key, parent=remap.get(s.parent, -1) if s.parent >= 0 else -1,
                        fork=s.fork, length=s.length, cached=s.cached))
    t = Tree(segs=segs, n_requests=1)
    return t, chain


def random_tree(rng: np.random.Generator, n_requests: int = 3, max_depth: int = 3,
                max_fanout: int = 3, max_len: int = 40, p_internal_fork: float = 0.3,
                p_cached_root: float = 0.0, max_cached: int = 48) -> Tree:
    """Small random rounds for brute-force and parity tests.

    Forks may fall inside a parent (not only at its end), lengths are ragged,
    and a request may start from a cached history.
    """
    reqs = []
    for _ in range(n_requests):
        nodes = []
        if rng.random() < p_cached_root:
            h = int(rng.integers(1, max_cached + 1))
            nodes.append((-1, 0, h, True))
            nodes.append((0, h, int(rng.integers(1, max_len + 1))))
            frontier = [(1, 1)]
        else:
            nodes.append((-1, 0, int(rng.integers(1, max_len + 1))))
            frontier = [(0, 0)]
        while frontier:
            idx, d = frontier.pop(0)
            if d + 1 > max_depth:
                continue
            nkids = int(rng.integers(0 if d > 0 else 1, max_fanout + 1))
            plen = nodes[idx][2]
            for _ in range(nkids):
                if rng.random() < p_internal_fork:
                    f = int(rng.integers(0, plen + 1))
                else:
                    f = plen
                nodes.append((idx, f, int(rng.integers(1, max_len + 1))))
                frontier.append((len(nodes) - 1, d + 1))
        reqs.append(nodes)
    return build_tree(reqs)
