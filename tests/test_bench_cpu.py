"""The benchmark's work counts, on trees small enough to count by hand: the
visible (query, key) pairs behind the attention FLOP figure, the pairs under
the sliding-window and two-way rules, and the GDN pass's algorithmic bytes."""
from types import SimpleNamespace

import bench
from workloads import build_tree

# a 10-token root, a 3-token child forked at its end, a 2-token child forked
# after 4 tokens
TREE = [[(-1, 0, 10), (0, None, 3), (0, 4, 2)]]


def test_visible_pairs_by_hand():
    t = build_tree(TREE).flatten()
    root = sum(i + 1 for i in range(10))                 # positions 0..9
    end_child = sum(10 + i + 1 for i in range(3))        # positions 10..12
    mid_child = sum(4 + i + 1 for i in range(2))         # positions 4..5
    assert bench.visible_pairs(t) == root + end_child + mid_child == 102


def test_rule_pairs_by_hand():
    t = build_tree(TREE).flatten()
    # window W = 3: every row sees min(position + 1, 3) keys
    w3 = sum(min(i + 1, 3) for i in range(10)) + 3 * 3 + sum(min(4 + i + 1, 3) for i in range(2))
    assert bench.rule_pairs(t, 1, 3) == w3
    # two-way: a row sees its ancestors' prefix and its whole own segment
    two = 10 * 10 + 3 * (10 + 3) + 2 * (4 + 2)
    assert bench.rule_pairs(t, 2) == two
    # a window wider than every path is the causal count
    assert bench.rule_pairs(t, 1, 1000) == bench.visible_pairs(t)


def test_gdn_bytes_by_hand():
    t = build_tree(TREE).flatten()
    sh = SimpleNamespace(Hk=2, Hv=4, dk=8, dv=16)
    per_tok = 2 * 2 * 8 * 2 + 2 * 4 * 16 * 2 + 2 * 4 * 4
    state = 4 * 16 * 8 * 4
    # two distinct fork points, each written once and read by its one child
    assert bench.gdn_bytes(t, sh, 2) == 15 * per_tok + 4 * state
    # siblings at one fork point share its single write and its single read
    # (the broadcast: both enter from the same state by index)
    t2 = build_tree([[(-1, 0, 10), (0, None, 3), (0, None, 2)]]).flatten()
    assert bench.gdn_bytes(t2, sh, 2) == 15 * per_tok + 2 * state
    assert bench.gdn_forks(t2) == (1, 2, 0)
    # a root resumed from a cached history reads its state slot; the resume
    # step also writes it back and the checkpoint save copies it out
    t3 = build_tree([[(-1, 0, 7, True), (0, None, 5)]]).flatten()
    assert bench.gdn_bytes(t3, sh, 2) == 5 * per_tok + 1 * state
    assert bench.gdn_bytes(t3, sh, 2, resumed_save=True) == 5 * per_tok + 4 * state


def test_path_tokens_by_hand():
    # the two leaves' whole paths: 10 + 3 and 4 + 2 positions; the root is no leaf
    t = build_tree(TREE).flatten()
    assert bench.path_tokens(t) == 13 + 6
    # a lone root is its own leaf; a cached history counts toward its leaf's path
    assert bench.path_tokens(build_tree([[(-1, 0, 7)]]).flatten()) == 7
    assert bench.path_tokens(build_tree([[(-1, 0, 7, True), (0, None, 5)]]).flatten()) == 12


def test_more_than_one_gpu_is_refused():
    # one GPU only: asked for more, the bench says so in its one line and exits
    import json
    import subprocess
    import sys
    from pathlib import Path

    root = Path(bench.__file__).resolve().parent
    r = subprocess.run([sys.executable, str(root / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120, cwd=root)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_kv_bytes_by_hand():
    # keys and values of every stream token, read once and written once
    t = build_tree(TREE).flatten()
    sh = SimpleNamespace(Hkv=2, d=8)
    assert bench.kv_bytes(t, sh, 2) == 4 * 15 * 2 * 8 * 2


def test_path_work_by_hand():
    # live rows and cached history rows on each leaf's isolated path
    t = build_tree(TREE).flatten()
    assert bench.path_work(t, 1) == (13, 0) and bench.path_work(t, 2) == (6, 0)
    t3 = build_tree([[(-1, 0, 7, True), (0, None, 5), (1, 2, 4)]]).flatten()
    assert bench.path_work(t3, 2) == (6, 7)
