"""Forked short causal convolution (gdn_conv_forward) against the fp64 oracle:
fp32 max-abs 1e-4; bf16 max-abs 2e-2 and mean-abs 2e-3; the saved windows
bit-exact (they are copies of inputs); and batch invariance bitwise (a leaf
alone equals the leaf inside the round).  Cached histories bring the window
the oracle computes for them as live roots (Flide section 3.4: a checkpoint
keeps the convolution window), so a resumed round is compared with the full
pass over the history."""
import numpy as np
import pytest
import torch

import gated_deltanet_amd as fk
import oracle
from workloads import build_tree, draw_conv, make_config, random_tree, subtree_path

pytestmark = pytest.mark.gpu
TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 2e-3)}


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.cuda()


def _f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _hist_windows(tree, cin):
    """Window of every cached segment: the oracle's window of the cached
    chain run as a live sequence (cached segments here are roots, or
    children of cached segments forked at their end)."""
    cached = [i for i, s in enumerate(tree.segs) if s.cached]
    W = cin.W
    if not cached or W == 1:
        return np.zeros((max(len(cached), 1), max(W - 1, 1), cin.C)), cached
    # cached rows as one live round: same parents and forks, every cached
    # segment a live segment with a state_out slot
    idx = {s: j for j, s in enumerate(cached)}
    par = np.array([idx[tree.segs[s].parent] if tree.segs[s].parent >= 0 else -1 for s in cached], np.int32)
    fork = np.array([tree.segs[s].fork if tree.segs[s].parent >= 0 else 0 for s in cached], np.int32)
    lens = [tree.segs[s].length for s in cached]
    tok = np.concatenate([np.full(n, j, np.int32) for j, n in enumerate(lens)])
    hx = cin.f64(True)
    rows = np.concatenate([hx[cin.hist_off[s]: cin.hist_off[s] + tree.segs[s].length] for s in cached])
    _, win = oracle.conv(tok, par, fork, np.zeros(len(cached), np.int32), np.zeros(len(cached) + 1, np.int64),
                         rows, None, cin.w, seg_state_out=np.arange(len(cached), dtype=np.int32),
                         n_state_out=len(cached))
    return win, cached


def _raw_window(win64, dtype):
    if dtype == "bf16":
        from workloads.tensors import to_bf16
        return to_bf16(win64)
    return win64.astype(np.float32)


class ConvRound:
    def __init__(self, tree, cin, all_state_out=True):
        self.tree, self.cin = tree, cin
        ts, par, fk_, cl = tree.arrays()
        S = tree.S
        cached = [i for i, s in enumerate(tree.segs) if s.cached]
        live = [i for i in range(S) if not tree.segs[i].cached]
        ssi = np.full(S, -1, np.int32)
        ssi[cached] = np.arange(len(cached))
        sso = np.full(S, -1, np.int32)
        if all_state_out:
            sso[live] = np.arange(len(live))
        self.ssi, self.sso = ssi, sso
        self.n_out = len(live) if all_state_out else 0
        hist_pages, nxt = {}, 0
        for s in cached:
            n = -(-tree.segs[s].length // 16)
            hist_pages[s] = list(range(nxt, nxt + n))
            nxt += n
        n_pages = max(nxt + sum(-(-tree.segs[i].length // 16) for i in live), 1)
        self.plan = fk.plan_round(ts, par, fk_, cl, cached_pages=hist_pages, first_page=nxt, n_pages=n_pages,
                                  seg_state_in=ssi, seg_state_out=sso, n_state_in=len(cached),
                                  n_state_out=self.n_out)
        self.meta = self.plan.meta
        self.ws = fk.alloc_workspace(self.meta)
        win64, _ = _hist_windows(tree, cin)
        self.window_in = _dev(_raw_window(win64, cin.dtype), cin.dtype) if cached and cin.W > 1 else None
        self.window_out = None
        if self.n_out and cin.W > 1:
            dt = torch.bfloat16 if cin.dtype == "bf16" else torch.float32
            self.window_out = torch.full((self.n_out, cin.W - 1, cin.C), float("nan"), dtype=dt, device="cuda")
        self.x = _dev(cin.x, cin.dtype)
        self.w = torch.from_numpy(cin.w).cuda()

    def run(self):
        fk.fk_tree_build(self.meta, self.ws)
        y = fk.gdn_conv_forward(self.meta, self.x, self.w, self.ws, window_in=self.window_in,
                                window_out=self.window_out)
        assert fk.fk_read_status(self.ws) == 0
        return y


def _oracle(tree, cin, sso, n_out):
    ts, par, fk_, cl = tree.arrays()
    return oracle.conv(ts, par, fk_, cl, cin.hist_off, cin.f64(), cin.f64(True), cin.w,
                       seg_state_out=sso, n_state_out=n_out)


def _check(tree, cin, label):
    r = ConvRound(tree, cin)
    y = _f64(r.run())
    ref, win_ref = _oracle(tree, cin, r.sso, r.n_out)
    assert np.isfinite(y).all()
    d = np.abs(y - ref)
    mx, mean = TOL[cin.dtype]
    print(f"  {label}: max {d.max():.2e} mean {d.mean():.2e}", flush=True)
    assert d.max() <= mx and d.mean() <= mean, (label, d.max(), d.mean())
    if r.window_out is not None:
        assert np.array_equal(_f64(r.window_out), win_ref), label
    return r, y


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_conv_random_trees(dtype):
    for seed in range(12):
        rng = np.random.default_rng(4100 + seed)
        t = random_tree(rng, p_cached_root=0.5, p_internal_fork=0.5, max_len=70, max_cached=40)
        if seed % 2:
            live = [i for i, s in enumerate(t.segs) if not s.cached]
            t.flatten(list(rng.permutation(live)))
        else:
            t.flatten()
        W = [4, 1, 2, 3, 5, 8][seed % 6]
        C = [64, 24, 2056, 512][seed % 4] if dtype == "bf16" else [64, 20, 1028, 512][seed % 4]
        cin = draw_conv(t, C, W, 300 + seed, dtype)
        print(f"[conv {dtype}] seed {seed} T={t.T} S={t.S} C={C} W={W}", flush=True)
        _check(t, cin, f"seed {seed}")


def test_conv_edges():
    """Halos that cross several ancestors: chains of one-token segments,
    forks at offset 0, a cached history shorter than the window, a fork at a
    tile boundary, one-token branches."""
    trees = [
        build_tree([[(-1, 0, 1)] + [(i, None, 1) for i in range(7)]]),                  # depth-8 chain of 1s
        build_tree([[(-1, 0, 2, True), (0, None, 1), (1, None, 1), (2, 0, 3), (3, 1, 20)]]),
        build_tree([[(-1, 0, 16), (0, 16, 5), (0, 0, 4), (0, 15, 17), (1, 0, 1)]]),
        build_tree([[(-1, 0, 1, True), (0, None, 2, True), (1, None, 1), (2, None, 33)],
                    [(-1, 0, 40), (0, 1, 1), (0, 40, 1)]]),
    ]
    for i, t in enumerate(trees):
        t.flatten()
        for W in (4, 8):
            for dtype in ("f32", "bf16"):
                cin = draw_conv(t, 256, W, 77 + i, dtype)
                print(f"[conv edge] tree {i} W={W} {dtype}", flush=True)
                _check(t, cin, f"edge {i} W={W} {dtype}")


def test_conv_batch_invariance():
    """Every leaf alone (its root-to-leaf chain, same boundaries) gives the
    same bits as inside the round; a permuted stream gives the same bits."""
    rng = np.random.default_rng(4242)
    t = random_tree(rng, n_requests=4, p_cached_root=0.5, p_internal_fork=0.4, max_len=60).flatten()
    C, W = 1024, 4
    cin = draw_conv(t, C, W, 55, "bf16")
    r = ConvRound(t, cin)
    y = _f64(r.run())
    starts = {}
    for x, s in enumerate(t.tok_seg):
        starts.setdefault(int(s), x)
    leaves = [i for i, s in enumerate(t.segs) if not s.cached and not t.children(i)]
    for leaf in leaves:
        sub, chain = subtree_path(t, leaf)
        sub.flatten()
        cs = draw_conv(sub, C, W, 55, "bf16", request_streams=[t.segs[leaf].request])
        ra = ConvRound(sub, cs)
        ya = _f64(ra.run())
        sub_starts = {}
        for x, s in enumerate(sub.tok_seg):
            sub_starts.setdefault(int(s), x)
        for new, old in enumerate(chain):
            if t.segs[old].cached:
                continue
            n = t.segs[old].length
            assert np.array_equal(ya[sub_starts[new]: sub_starts[new] + n], y[starts[old]: starts[old] + n]), leaf
    live = [i for i, s in enumerate(t.segs) if not s.cached]
    tp = random_tree(np.random.default_rng(4242), n_requests=4, p_cached_root=0.5, p_internal_fork=0.4,
                     max_len=60).flatten(list(np.random.default_rng(1).permutation(live)))
    cp = draw_conv(tp, C, W, 55, "bf16")
    yp = _f64(ConvRound(tp, cp).run())
    pst = {}
    for x, s in enumerate(tp.tok_seg):
        pst.setdefault(int(s), x)
    for s in live:
        n = t.segs[s].length
        assert np.array_equal(yp[pst[s]: pst[s] + n], y[starts[s]: starts[s] + n])


@pytest.mark.parametrize("which,C", [(1, 6144), (2, 1024), (3, 512)])
def test_conv_configs(which, C):
    """Full-size trees of the mixture (q|k|v channels of its GDN layer), the
    depth-3 fan-out and the 32k-trunk workloads, every token."""
    cfg, t = make_config(which)
    cin = draw_conv(t, C, 4, cfg.seed, "bf16")
    print(f"[conv config {which}] T={t.T} C={C}", flush=True)
    _check(t, cin, f"config {which}")
