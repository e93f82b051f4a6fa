"""Stored values from the pages (tests/golden/, each file cites its source)."""
import os

import numpy as np

import oracle
from workloads import build_tree

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _kv(name):
    out = {}
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split()
            out[k] = int(v)
    return out


def test_forkserve_fanout_token_counts():
    g = _kv("forkserve_fanout.txt")
    nodes = [(-1, 0, g["trunk"])] + [(0, None, g["residual"])] * g["fanout"]
    t = build_tree([nodes] * g["sessions"]).flatten()
    ix = oracle.index(*t.arrays())
    # state once plus every question once: the flat stream
    assert t.T == g["alias_prefill_tokens"]
    # every question as its own sequence: sum over leaves of (pos0 + len)
    leaves = t.leaves()
    iso = int(sum(ix["seg_pos0"][s] + ix["seg_len"][s] for s in leaves))
    assert iso == g["apc_prefill_tokens"]
    # K/V held once per page-aligned segment (children alias the trunk's pages)
    P = g["page"]
    pages = int(sum(-(-ix["seg_len"][s] // P) for s in range(t.S)))
    assert pages * P == g["alias_peak_kv_tokens"]


def test_visible_pair_closed_forms():
    g = _kv("visible_pairs.txt")
    trees = {
        "tiny_48_6_8_10": [[(-1, 0, 48), (0, None, 6), (0, None, 8), (0, None, 10)]],
        "long_4x32768_16x64": [[(-1, 0, 32768)] + [(0, None, 64)] * 16] * 4,
    }
    nodes = [(-1, 0, 4096)]
    for _ in range(4):
        nodes.append((0, None, 256))
        p = len(nodes) - 1
        nodes += [(p, None, 32)] * 4
    trees["fanout_10x4096_4x256_4x32"] = [nodes] * 10
    for name, reqs in trees.items():
        t = build_tree(reqs).flatten()
        ix = oracle.index(*t.arrays())
        assert int((ix["tok_pos"].astype(np.int64) + 1).sum()) == g[name], name
