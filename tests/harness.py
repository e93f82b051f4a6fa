"""Run a seeded workload through the HIP library (via the C-ABI binding) and
through the oracle, on the same inputs.

Cached segments get their history K/V the way a real resume does: a history
round (the cached segments as live roots) appends them into pages first, and
the main round then names those pages.  Their recurrent states come from
``state_in`` (a seeded random state, or a checkpoint of the GPU's own pass).
"""
from __future__ import annotations

import functools

import numpy as np
import torch

import gated_deltanet_amd as fk
import oracle
from workloads import make_config
from workloads.tensors import ACT, draw_inputs


def dev_tensor(inp, name, hist=False, device="cuda"):
    x = (inp.hist if hist else inp.raw)[name]
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.bfloat16) if hasattr(t, "view") else t
    return t.to(device)


@functools.lru_cache(maxsize=None)
def config_inputs(i: int):
    """(config, host-drawn inputs) of workload i, drawn once per test session
    (the long-context round takes about a minute to draw)."""
    cfg, t = make_config(i)
    return cfg, draw_inputs(t, cfg.shapes, cfg.seed, cfg.dtype, cfg.mu_a)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def state_slots(tree):
    """state_in slot per cached segment (in index order); state_out slot per
    live segment (all of them, so tests can read every final state)."""
    S = tree.S
    cached = [i for i, s in enumerate(tree.segs) if s.cached]
    ssi = np.full(S, -1, np.int32)
    ssi[cached] = np.arange(len(cached))
    sso = np.full(S, -1, np.int32)
    live = [i for i in range(S) if i not in set(cached)]
    sso[live] = np.arange(len(live))
    return ssi, sso, len(cached), len(live)


class GpuRound:
    """One round on the GPU: plan, history pages, build, attention, GDN."""

    def __init__(self, inp, state_in_np=None, n_pool_extra=0, device="cuda", want_state_out=True,
                 pool_fill=0.0):
        self.inp = inp
        tree = inp.tree
        sh = inp.shapes
        self.device = device
        ts, par, fk_, cl = tree.arrays()
        ssi, sso, n_in, n_out = state_slots(tree)
        if not want_state_out:
            sso[:] = -1
            n_out = 0
        self.ssi, self.sso, self.n_in, self.n_out = ssi, sso, n_in, n_out
        dt = torch.bfloat16 if inp.dtype == "bf16" else torch.float32
        self.dt = dt
        # pages: history pages first, then this round's live pages
        cached = [i for i, s in enumerate(tree.segs) if s.cached]
        hist_pages = {}
        nxt = 0
        for s in cached:
            n = -(-tree.segs[s].length // 16)
            hist_pages[s] = list(range(nxt, nxt + n))
            nxt += n
        live_pages = sum(-(-tree.segs[i].length // 16) for i in range(tree.S) if not tree.segs[i].cached)
        self.n_pages = max(nxt + live_pages + n_pool_extra, 1)
        self.k_pool = torch.full((self.n_pages, sh.Hkv, 16, sh.d), pool_fill, dtype=dt, device=device)
        self.v_pool = torch.full((self.n_pages, sh.Hkv, sh.d, 16), pool_fill, dtype=dt, device=device)
        if cached:
            # history round: each cached segment as a live root of its own
            hts = np.concatenate([np.full(tree.segs[s].length, j, np.int32) for j, s in enumerate(cached)])
            hplan = fk.plan_round(hts, np.full(len(cached), -1), np.zeros(len(cached)),
                                  np.zeros(len(cached)), first_page=0, n_pages=self.n_pages,
                                  device=device)
            hws = fk.alloc_workspace(hplan.meta, device=device)
            fk.fk_tree_build(hplan.meta, hws)
            fk.kv_append(hplan.meta, dev_tensor(inp, "ak", True), dev_tensor(inp, "av", True),
                         self.k_pool, self.v_pool, hws)
            assert fk.fk_read_status(hws) == 0
        self.plan = fk.plan_round(ts, par, fk_, cl, cached_pages=hist_pages, first_page=nxt,
                                  n_pages=self.n_pages, seg_state_in=ssi, seg_state_out=sso,
                                  n_state_in=n_in, n_state_out=n_out, device=device)
        self.meta = self.plan.meta
        self.ws = fk.alloc_workspace(self.meta, sh.Hv, sh.dk, sh.dv, device=device)
        self.state_in = None
        if n_in:
            st = state_in_np if state_in_np is not None else np.zeros((n_in, sh.Hv, sh.dv, sh.dk))
            self.state_in = torch.from_numpy(np.ascontiguousarray(st, np.float32)).to(device)
        self.state_out = torch.full((max(n_out, 1), sh.Hv, sh.dv, sh.dk), float("nan"),
                                    dtype=torch.float32, device=device)
        self.x = {n: dev_tensor(inp, n) for n in inp.raw}

    def build(self):
        fk.fk_tree_build(self.meta, self.ws)
        return self

    def status(self):
        return fk.fk_read_status(self.ws)

    def attention(self, scale=None, rule=None, window=0):
        if rule is None:
            return fk.fork_attn_forward(self.meta, self.x["aq"], self.x["ak"], self.x["av"], self.k_pool,
                                        self.v_pool, self.ws, scale=scale)
        return fk.fork_attn_forward_rule(self.meta, self.x["aq"], self.x["ak"], self.x["av"], self.k_pool,
                                         self.v_pool, self.ws, rule, window, scale=scale)

    def gdn(self):
        return fk.gdn_fork_forward(self.meta, self.x["gq"], self.x["gk"], self.x["gv"], self.x["ga"],
                                   self.x["gb"], self.ws, state_in=self.state_in,
                                   state_out=self.state_out if self.n_out else None)


def stratified_rows(tree, trunk_every=64):
    """First and last row of every 16-token tile of every non-root segment;
    first and last row of every ``trunk_every``-th tile of a root segment (and
    of its last tile)."""
    sel = np.zeros(tree.T, bool)
    starts = {}
    for x, s in enumerate(tree.tok_seg):
        starts.setdefault(int(s), x)
    for s, x0 in starts.items():
        seg = tree.segs[s]
        root = seg.parent < 0 or tree.segs[seg.parent].cached
        n_tiles = -(-seg.length // 16)
        tiles = set(range(0, n_tiles, trunk_every)) | {n_tiles - 1} if root else range(n_tiles)
        for j in tiles:
            sel[x0 + 16 * j] = True
            sel[x0 + min(16 * j + 15, seg.length - 1)] = True
    return sel


def oracle_attention(inp, mode=1, tok_sel=None, scale=None, rule=0, window=0, head_sel=None):
    ts, par, fk_, cl = inp.tree.arrays()
    d = inp.shapes.d
    return oracle.attention(ts, par, fk_, cl, inp.hist_off, inp.f64("aq"), inp.f64("ak"), inp.f64("av"),
                            inp.f64("ak", True), inp.f64("av", True),
                            scale if scale is not None else 1 / np.sqrt(d), mode=mode, tok_sel=tok_sel,
                            head_sel=head_sel, rule=rule, window=window)[0]


def oracle_gdn(inp, state_in=None, mode=1, head_sel=None):
    ts, par, fk_, cl = inp.tree.arrays()
    ssi, sso, n_in, n_out = state_slots(inp.tree)
    o, st, _ = oracle.gdn(ts, par, fk_, cl, inp.f64("gq"), inp.f64("gk"), inp.f64("gv"), inp.f64("ga"),
                          inp.f64("gb"), state_in=state_in, seg_state_in=ssi, seg_state_out=sso,
                          n_state_out=n_out, mode=mode, head_sel=head_sel)
    return o, st
