#!/usr/bin/env python3
"""Benchmark one forked pass of the hot path on one MI355X.

A step is one pass over one round of synthetic decision requests: the
tree-metadata build, the paged K/V append, ForkAttention over the round
(GQA softmax attention, every branch seeing only its ancestry), and the
forked Gated DeltaNet layer (trunk once, children from the fork-point state
by index); on the resume workload also the checkpoint resume and save.

Default workload (the headline line): the expanding-history resume round --
64 requests, each resumed from a checkpoint (fp32 GDN state + 16,384-token
paged K/V), 1,024 new history tokens, then mixed trees of 32-token question
branches (depth 1-3, fan-out 2-8); bf16, attention 32 q / 4 kv heads d 128,
GDN 16 k / 32 v heads 128 x 128.  The same run also measures the 16-request
mixture, the depth-3 agent fan-out and the 32k-token long context
(``--also``), each reported under ``configs`` with its own rooflines and CPU
oracle baseline.  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config 4] [--also 1,2,3]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "branch tokens/sec (fork attn + GDN) at 1 MI355X; % of MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=4, help="headline workload index (1-4)")
    ap.add_argument("--also", default="1,2,3",
                    help="further workloads measured in the same run (comma list, '' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next-rows", action="store_true",
                    help="skip the rows beyond the step (conv, rules, readout, projection GEMM)")
    ap.add_argument("--cpu-requests", type=int, default=16,
                    help="requests of the mixture in its CPU oracle sample")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of replays of the step captured as a HIP graph")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain copy of 256 MiB (gdn_checkpoint_save) before timing, so a "
                         "counter run can scale FETCH_SIZE / WRITE_SIZE to bytes")
    return ap.parse_args()


CSRC = os.path.join(ROOT, "gated_deltanet_amd", "csrc")
SLUG = {1: "mixture", 2: "fanout", 3: "long_context", 4: "resume"}
# kernel family -> (profile name, source file whose hash the counter summary records)
TRAFFIC_KERNELS = {"attention": ("attn_bf16", "attn_bf16.hip"), "gdn": ("gdn_bf16", "gdn_bf16.hip"),
                   "kv_append": ("kv_append", "kv_append.hip")}


def kernel_hash(path: str) -> str:
    import hashlib
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_file(kernel: str, config: int) -> str:
    return os.path.join(ROOT, "profiles", f"{TRAFFIC_KERNELS[kernel][0]}_{SLUG.get(config, config)}_traffic.txt")


def measured_traffic(kernel: str, config: int):
    """HBM bytes per launch (per step for the GDN phase) of a kernel family from
    the committed counter summary, or None when it is missing, for another
    workload, or the kernel source changed since the counters were taken."""
    path = traffic_file(kernel, config)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        parts = line.split()
        if len(parts) == 2 and not line.startswith("#"):
            kv[parts[0]] = parts[1]
    src = os.path.join(CSRC, TRAFFIC_KERNELS[kernel][1])
    if kv.get("kernel_sha256_16") != kernel_hash(src) or kv.get("config") != str(config):
        return None
    return float(kv["bytes_per_launch"])


def calibrate_copy():
    """One plain 256 MiB device copy through the checkpoint-save kernel."""
    import torch
    import gated_deltanet_amd as fk
    src = torch.ones((1, 4096, 128, 128), dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src[0])
    fk.gdn_checkpoint_save(src, 0, dst)
    torch.cuda.synchronize()
    return src.numel() * 4


def measured_peaks():
    """What this device sustains, reported next to the published peaks (the
    roofline fractions use the published ones): a plain 512 MiB copy through
    the checkpoint-save kernel (read + write) and the dense bf16 MFMA loop."""
    import torch
    import gated_deltanet_amd as fk
    src = torch.ones((1, 8192, 128, 128), dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src[0])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        fk.gdn_checkpoint_save(src, 0, dst)
    e0.record()
    for _ in range(10):
        fk.gdn_checkpoint_save(src, 0, dst)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * src.numel() * 4 * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    n_wg = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(n_wg, dtype=torch.float32, device="cuda")
    fk.fk_peak_mfma_bf16(n_wg, 256, sink)
    e0.record()
    flops = sum(fk.fk_peak_mfma_bf16(n_wg, 4096, sink) for _ in range(5))
    e1.record()
    torch.cuda.synchronize()
    tf = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    return {"hbm_copy_GBs": copy_gbs, "mfma_bf16_TFLOPs": tf,
            "published": {"hbm_GBs": PEAK_HBM_GBS, "mfma_bf16_TFLOPs": PEAK_BF16_TFLOPS},
            "how": "512 MiB copy (checkpoint-save kernel, read + write bytes); eight independent "
                   "32x32x16 bf16 MFMA chains per wave, two waves per SIMD, register operands"}


def path_tokens(tree) -> int:
    """Isolated-pass work the method avoids: every leaf's whole root-to-leaf
    path (positions 0 .. pos0 + len - 1), summed over live leaves."""
    tot = 0
    for i, sg in enumerate(tree.segs):
        if sg.cached or any(not tree.segs[c].cached for c in tree.children(i)):
            continue
        pos0, j = 0, i
        while tree.segs[j].parent >= 0:
            pos0 += tree.segs[j].fork
            j = tree.segs[j].parent
        tot += pos0 + sg.length
    return tot


def visible_pairs(tree) -> int:
    """Visible (query, key) pairs per attention head: sum over live segments
    of len*pos0 + len(len+1)/2 (positions continue from the fork)."""
    pos0 = np.zeros(tree.S, np.int64)
    for i in range(tree.S):
        acc, j = 0, i
        while tree.segs[j].parent >= 0:
            acc += tree.segs[j].fork
            j = tree.segs[j].parent
        pos0[i] = acc
    tot = 0
    for i, s in enumerate(tree.segs):
        if not s.cached:
            L = s.length
            tot += L * int(pos0[i]) + L * (L + 1) // 2
    return tot


class Step:
    """One step = four phases on torch's current stream: build (on the resume
    workload: resume + build), K/V append, ForkAttention, forked GDN (on the
    resume workload: + checkpoint save).  GDN reads nothing the append or the
    attention write, so the overlapped form runs the GDN phase on a second
    stream, forked after the build and joined at the end; its outputs are
    bit-identical to the serial form's."""

    def step(self, ev=None):
        """Serial; with ``ev`` (five events) the phase boundaries are recorded."""
        for i, phase in enumerate((self.build, self.append, self.attention, self.gdn)):
            if ev:
                ev[i].record()
            phase()
        if ev:
            ev[4].record()

    def step_overlapped(self):
        torch = self.torch
        if not hasattr(self, "_side"):
            self._side = torch.cuda.Stream()   # default priority
        self.build()
        cur = torch.cuda.current_stream()
        self._side.wait_stream(cur)
        with torch.cuda.stream(self._side):
            self.gdn()
        self.append()
        self.attention()
        cur.wait_stream(self._side)


def pad_rows(x: dict, rows: int) -> dict:
    """Stream tensors padded with zero rows up to a bucket's capacity."""
    import torch

    out = {}
    for n, t in x.items():
        p = torch.zeros((rows,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
        p[:t.shape[0]] = t
        out[n] = p
    return out


class Workload(Step):
    """A config's round resident on the GPU, ready to step.  bf16 inputs are
    drawn on the GPU (seeded, the workload recipe, torch's generator); the
    fp32 tiny request uses the host generator."""

    def __init__(self, index: int, device="cuda"):
        import torch

        import gated_deltanet_amd as fk
        from workloads import make_config
        from workloads.device import draw_stream
        from workloads.tensors import draw_inputs

        self.torch, self.fk = torch, fk
        cfg, tree = make_config(index)
        assert not any(s.cached for s in tree.segs), "the resume workload uses ResumeWorkload"
        self.cfg, self.tree = cfg, tree
        sh = cfg.shapes
        self.sh = sh
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        ts, par, fkk, cl = tree.arrays()
        # the round in the smallest capacity bucket that holds it (tail
        # padding, unused segment slots): the graph replayed below is that
        # bucket's, valid for any round that fits it
        self.bucket = fk.bucket_for(tree.T, tree.S, *fk.capacities(par, fkk, cl))
        if cfg.dtype == "bf16":
            x = draw_stream(tree.T, sh, cfg.seed * 7 + 2, cfg.mu_a, device)
        else:
            inp = draw_inputs(tree, cfg.shapes, cfg.seed, cfg.dtype, cfg.mu_a)
            x = {n: torch.from_numpy(np.ascontiguousarray(inp.raw[n])).to(device) for n in inp.raw}
            del inp
        self.x = pad_rows(x, self.bucket.T)
        sso = np.full(tree.S, -1, np.int32)
        self.plan = fk.plan_round(ts, par, fkk, cl, seg_state_out=sso, n_state_out=0, bucket=self.bucket,
                                  device=device)
        self.meta = self.plan.meta
        self.ws = fk.alloc_workspace(self.meta, sh.Hv, sh.dk, sh.dv, device=device)
        n_pages = self.plan.n_pages
        self.k_pool = torch.zeros((n_pages, sh.Hkv, 16, sh.d), dtype=dt, device=device)
        self.v_pool = torch.zeros((n_pages, sh.Hkv, sh.d, 16), dtype=dt, device=device)
        self.attn_out = torch.zeros_like(self.x["aq"])   # padding rows stay zero
        self.gdn_out = torch.zeros_like(self.x["gv"])
        self.scale = sh.d ** -0.5
        self.gdn_ok = True

    def build(self):
        self.fk.fk_tree_build(self.meta, self.ws)

    def append(self):
        x = self.x
        self.fk.kv_append(self.meta, x["ak"], x["av"], self.k_pool, self.v_pool, self.ws)

    def attention(self):
        x = self.x
        self.fk.fork_attn_forward(self.meta, x["aq"], None, None, self.k_pool, self.v_pool, self.ws,
                                  scale=self.scale, out=self.attn_out)

    def gdn(self):
        fk, x = self.fk, self.x
        if self.gdn_ok:
            try:
                fk.gdn_fork_forward(self.meta, x["gq"], x["gk"], x["gv"], x["ga"], x["gb"], self.ws,
                                    out=self.gdn_out)
            except fk._lib.FkError as e:   # reported in the JSON line, never silently
                if e.name != "FK_E_UNSUPPORTED":
                    raise
                self.gdn_ok = False


class ResumeWorkload(Step):
    """The expanding-history workload: every request resumes from a checkpoint
    -- the fp32 GDN state and the 16,384-token paged K/V of its history, made
    by an untimed GPU pass over that history -- appends 1,024 new tokens and
    forks a mixed tree of 32-token branches.  A step resumes the saved
    states, runs the round, and saves the new roots' states for the next step.

    Inputs are drawn on the GPU (seeded); ``sampled`` requests instead use the
    host generator's values so an oracle can check them.
    """

    def __init__(self, device="cuda", sampled=()):
        import torch

        import gated_deltanet_amd as fk
        from workloads import make_config
        from workloads.device import draw_stream
        from workloads.tensors import SeedTree, draw_segment

        self.torch, self.fk = torch, fk
        cfg, tree = make_config(4)
        self.cfg, self.tree, self.sh = cfg, tree, cfg.shapes
        sh = cfg.shapes
        hist = [i for i, sg in enumerate(tree.segs) if sg.cached]
        self.hist = hist
        R, H = len(hist), tree.segs[hist[0]].length
        self.R, self.H = R, H
        # pass 1: every history as a live root, laid out request by request
        self.hx = draw_stream(R * H, sh, cfg.seed * 7 + 1, cfg.mu_a, device,
                              names=("ak", "av", "gq", "gk", "gv", "ga", "gb"))
        # the round: live stream in tree order, padded to its capacity bucket
        self.bucket = fk.bucket_for(tree.T, tree.S, *fk.capacities(*tree.arrays()[1:]))
        self.x = pad_rows(draw_stream(tree.T, sh, cfg.seed * 7 + 2, cfg.mu_a, device), self.bucket.T)
        starts, acc = {}, 0
        for sid in tree.order:
            starts[sid] = acc
            acc += tree.segs[sid].length
        self.starts = starts
        seeds = SeedTree(cfg.seed)

        def put(dst, t0, vals):
            for name, arr in vals.items():
                if name not in dst:
                    continue
                t = torch.from_numpy(np.ascontiguousarray(arr))
                if arr.dtype == np.uint16:
                    t = t.view(torch.bfloat16)
                dst[name][t0:t0 + len(arr)] = t.to(device)

        for r in sampled:
            for sid, sg in enumerate(tree.segs):
                if sg.request != r:
                    continue
                vals = draw_segment(seeds, r, sg.key, sg.length, sh, cfg.mu_a, "bf16")
                if sg.cached:
                    put(self.hx, hist.index(sid) * H, vals)
                else:
                    put(self.x, starts[sid], vals)
        n_hist_pages = R * H // 16
        n_pages = n_hist_pages + sum(-(-sg.length // 16) for sg in tree.segs if not sg.cached)
        ts, par, fkk, cl = tree.arrays()
        ssi = np.full(tree.S, -1, np.int32)
        sso = np.full(tree.S, -1, np.int32)
        cached_pages = {}
        for r, sid in enumerate(hist):
            ssi[sid] = r
            cached_pages[sid] = np.arange(r * (H // 16), (r + 1) * (H // 16))
            (root,) = tree.children(sid)
            sso[root] = r
        self.plan = fk.plan_round(ts, par, fkk, cl, cached_pages=cached_pages, first_page=n_hist_pages,
                                  n_pages=n_pages, seg_state_in=ssi, seg_state_out=sso, n_state_in=R,
                                  n_state_out=R, bucket=self.bucket, device=device)
        assert n_hist_pages + self.plan.pages_used == n_pages
        self.meta = self.plan.meta
        self.hplan = fk.plan_round(np.repeat(np.arange(R, dtype=np.int32), H), np.full(R, -1), np.zeros(R),
                                   np.zeros(R), first_page=0, n_pages=n_pages,
                                   seg_state_out=np.arange(R, dtype=np.int32), n_state_out=R, device=device)
        dt = torch.bfloat16
        self.k_pool = torch.zeros((n_pages, sh.Hkv, 16, sh.d), dtype=dt, device=device)
        self.v_pool = torch.zeros((n_pages, sh.Hkv, sh.d, 16), dtype=dt, device=device)
        st = (R, sh.Hv, sh.dv, sh.dk)
        self.state_in = torch.zeros(st, dtype=torch.float32, device=device)
        self.state_out = torch.zeros(st, dtype=torch.float32, device=device)
        self.ckpt = torch.zeros(st, dtype=torch.float32, device=device)
        self.ckpt_next = torch.zeros(st, dtype=torch.float32, device=device)
        self.attn_out = torch.zeros_like(self.x["aq"])   # padding rows stay zero
        self.gdn_out = torch.zeros_like(self.x["gv"])
        self.scale = sh.d ** -0.5
        self.ws = fk.alloc_workspace(self.meta, sh.Hv, sh.dk, sh.dv, device=device)

    def checkpoint(self):
        """Untimed pass 1: page the histories' K/V, run GDN over them, save."""
        fk, torch, sh = self.fk, self.torch, self.sh
        hws = fk.alloc_workspace(self.hplan.meta, sh.Hv, sh.dk, sh.dv)
        fk.fk_tree_build(self.hplan.meta, hws)
        fk.kv_append(self.hplan.meta, self.hx["ak"], self.hx["av"], self.k_pool, self.v_pool, hws)
        hst = torch.empty((self.R, sh.Hv, sh.dv, sh.dk), dtype=torch.float32, device="cuda")
        fk.gdn_fork_forward(self.hplan.meta, self.hx["gq"], self.hx["gk"], self.hx["gv"], self.hx["ga"],
                            self.hx["gb"], hws, state_out=hst)
        assert fk.fk_read_status(hws) == 0
        fk.gdn_checkpoint_save(hst, 0, self.ckpt, count=self.R)
        torch.cuda.synchronize()
        del hws, hst

    def build(self):
        self.fk.gdn_checkpoint_resume(self.ckpt, self.state_in, 0, count=self.R)
        self.fk.fk_tree_build(self.meta, self.ws)

    def append(self):
        x = self.x
        self.fk.kv_append(self.meta, x["ak"], x["av"], self.k_pool, self.v_pool, self.ws)

    def attention(self):
        x = self.x
        self.fk.fork_attn_forward(self.meta, x["aq"], None, None, self.k_pool, self.v_pool, self.ws,
                                  scale=self.scale, out=self.attn_out)

    def gdn(self):
        fk, x = self.fk, self.x
        fk.gdn_fork_forward(self.meta, x["gq"], x["gk"], x["gv"], x["ga"], x["gb"], self.ws,
                            state_in=self.state_in, state_out=self.state_out, out=self.gdn_out)
        fk.gdn_checkpoint_save(self.state_out, 0, self.ckpt_next, count=self.R)


def gdn_forks(tree):
    """(distinct fork points between live segments, children entering from
    them, roots resumed from a cached history)."""
    forks, children, resumed = set(), 0, 0
    for s in tree.segs:
        if s.cached or s.parent < 0:
            continue
        if tree.segs[s.parent].cached:
            resumed += 1
        else:
            forks.add((s.parent, s.fork))
            children += 1
    return len(forks), children, resumed


def gdn_bytes(tree, sh, elem: int, resumed_save: bool = False) -> int:
    """Algorithmic HBM bytes of one forked GDN pass: q and k (Hk heads) and v
    read once, o written once, a and b read once (fp32); each fork-point
    state written once and read once (the broadcast: children enter from it
    by index); each resumed root reads its state_in slot, and with
    ``resumed_save`` (the resume workload's step) also writes its state_out
    slot, which the checkpoint save then reads and copies out."""
    per_tok = 2 * sh.Hk * sh.dk * elem + 2 * sh.Hv * sh.dv * elem + 2 * sh.Hv * 4
    state = sh.Hv * sh.dv * sh.dk * 4
    n_forks, _, resumed = gdn_forks(tree)
    n_states = 2 * n_forks + resumed + (3 * resumed if resumed_save else 0)
    return tree.T * per_tok + n_states * state


def kv_bytes(tree, sh, elem: int) -> int:
    """Algorithmic HBM bytes of the K/V append: the stream's keys and values
    read once and written once into their pages."""
    return 4 * tree.T * sh.Hkv * sh.d * elem


def measure_conv(wl, steps: int, W: int = 4):
    """The forked short convolution in front of the GDN layer (a row beyond
    the step), timed on its own over the same round: channels = the q|k|v
    projections of the GDN layer (2 Hk dk + Hv dv), width 4, bf16, windows
    read for cached histories and written for every state_out slot.
    HBM-bound: algorithmic bytes = the input read once + the output written
    once (+ windows)."""
    torch, fk, sh, meta = wl.torch, wl.fk, wl.sh, wl.meta
    C = 2 * sh.Hk * sh.dk + sh.Hv * sh.dv
    T = wl.meta.T   # the bucket's stream capacity (padding rows are never read or written)
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.cfg.seed * 7 + 3)
    x = torch.empty((T, C), dtype=torch.bfloat16, device="cuda")
    for t0 in range(0, T, 1 << 14):
        x[t0:t0 + (1 << 14)] = torch.randn((min(1 << 14, T - t0), C), generator=g, device="cuda")
    w = (torch.rand((C, W), generator=g, device="cuda") * 2 - 1) / W ** 0.5
    win_in = torch.randn((max(meta.n_state_in, 1), W - 1, C), generator=g, device="cuda").to(torch.bfloat16)
    win_out = torch.empty((max(meta.n_state_out, 1), W - 1, C), dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)

    def run():
        fk.gdn_conv_forward(meta, x, w, wl.ws, window_in=win_in if meta.n_state_in else None,
                            window_out=win_out if meta.n_state_out else None, out=y)

    run()
    torch.cuda.synchronize()
    assert fk.fk_read_status(wl.ws) == 0, "conv reported an error"
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = 2.0 * wl.tree.T * C * 2 + (meta.n_state_in + meta.n_state_out) * (W - 1) * C * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "forked short conv (bf16)", "channels": C, "width": W, "ms": ms, "bound": "hbm",
            "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
            "algorithmic_bytes": nbytes}


def rule_pairs(tree, rule: int, window: int = 0) -> int:
    """Visible (query, key) pairs per head under a visibility rule: a row at
    position p sees min(p + 1, W) keys in a window of width W (its path holds
    every earlier position), and pos0 + len keys when its segment is read
    both ways."""
    pos0 = np.zeros(tree.S, np.int64)
    for i in range(tree.S):
        acc, j = 0, i
        while tree.segs[j].parent >= 0:
            acc += tree.segs[j].fork
            j = tree.segs[j].parent
        pos0[i] = acc
    tot = 0
    for i, sg in enumerate(tree.segs):
        if sg.cached:
            continue
        pos = pos0[i] + np.arange(sg.length, dtype=np.int64)
        tot += int(np.minimum(pos + 1, window).sum()) if rule == 1 else int(sg.length * (pos0[i] + sg.length))
    return tot


def measure_rule(wl, steps: int, rule: int, window: int = 0):
    """ForkAttention under another visibility rule (a row beyond the step),
    over the same round with its keys/values already paged; MFMA roofline on
    the rule's own visible pairs."""
    torch, fk, sh = wl.torch, wl.fk, wl.sh
    out = torch.empty_like(wl.attn_out)

    def run():
        fk.fork_attn_forward_rule(wl.meta, wl.x["aq"], None, None, wl.k_pool, wl.v_pool, wl.ws, rule, window,
                                  scale=wl.scale, out=out)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 4.0 * sh.d * sh.Hq * rule_pairs(wl.tree, rule, window)
    tf = flops / (ms * 1e-3) / 1e12
    name = f"sliding-window attention (W={window})" if rule == 1 else "two-way attention"
    return {"kernel": name + " (bf16 MFMA)", "ms": ms, "bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS, "algorithmic_flops": flops}


def measure_readout(wl, steps: int):
    """Selective readout (a row beyond the step): attention at the last token
    of every question only, the round's keys/values already paged.  Bound by
    streaming those rows' keys/values: algorithmic bytes = every key/value
    token visible to some selected row, read once, plus their queries and
    outputs."""
    torch, fk, sh, tree = wl.torch, wl.fk, wl.sh, wl.tree
    starts, acc = {}, 0
    for sid in tree.order:
        starts[sid] = acc
        acc += tree.segs[sid].length
    leaves = [i for i, sg in enumerate(tree.segs) if not sg.cached and not tree.children(i)]
    rows = np.array([starts[i] + tree.segs[i].length - 1 for i in leaves], np.int32)
    seen = {}                       # segment -> keys of it visible to some selected row
    for i in leaves:
        seen[i] = tree.segs[i].length
        c = i
        while tree.segs[c].parent >= 0:
            p = tree.segs[c].parent
            seen[p] = max(seen.get(p, 0), tree.segs[c].fork)
            c = p
    kv_tokens = sum(seen.values())
    rows_t = torch.from_numpy(rows).cuda()
    q_rows = wl.x["aq"][rows_t.long()].contiguous()
    out = torch.empty_like(q_rows)

    def run():
        fk.fork_attn_readout(wl.meta, q_rows, rows_t, wl.k_pool, wl.v_pool, wl.ws, scale=wl.scale, out=out)

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = float(kv_tokens * sh.Hkv * sh.d * 2 * 2 + 2 * len(rows) * sh.Hq * sh.d * 2)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": "selective readout (bf16)", "rows": len(rows), "ms": ms, "bound": "hbm", "achieved": gbs,
            "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "algorithmic_bytes": nbytes}


def measure_proj(wl, steps: int):
    """The fixed-order projection (a row beyond the step): the attention
    layer's output projection, width Hq d -> Hq d, over every stream row of
    the round (the attention output as x; w ~ N(0, 1/K), seeded), and over
    the readout rows only (the last token of every question, gathered through
    an index buffer).  MFMA-bound: 2 M N K flops."""
    torch, fk, sh, tree = wl.torch, wl.fk, wl.sh, wl.tree
    K = N = sh.Hq * sh.d
    g = torch.Generator(device="cuda")
    g.manual_seed(wl.cfg.seed * 7 + 5)
    w = (torch.randn((N, K), generator=g, device="cuda") * K ** -0.5).to(torch.bfloat16)
    x = wl.attn_out[:tree.T].view(tree.T, K)
    starts, acc = {}, 0
    for sid in tree.order:
        starts[sid] = acc
        acc += tree.segs[sid].length
    rows = torch.tensor([starts[i] + tree.segs[i].length - 1 for i in tree.leaves()], dtype=torch.int32,
                        device="cuda")
    y = torch.empty((tree.T, N), dtype=torch.bfloat16, device="cuda")
    yr = torch.empty((rows.numel(), N), dtype=torch.bfloat16, device="cuda")
    out = {}
    for name, fn, M in (("stream_rows", lambda: fk.fk_proj_gemm(x, w, out=y), tree.T),
                        ("readout_rows", lambda: fk.fk_proj_gemm(x, w, rows=rows, out=yr), rows.numel())):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        flops = 2.0 * M * N * K
        tf = flops / (ms * 1e-3) / 1e12
        out[name] = {"kernel": "fixed-order projection (bf16 MFMA)", "M": M, "K": K, "N": N, "ms": ms,
                     "bound": "mfma", "achieved": tf, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tf / PEAK_BF16_TFLOPS, "algorithmic_flops": flops}
    del y, yr, w
    return out


def host_cpu():
    """The host CPU the oracle ran on: model name and the CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "affinity_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline(index: int, n_req: int):
    """The fp64 oracle, as it stands, on a bounded sample of the same workload
    (branch tokens/s).  The mixture: its first ``n_req`` requests, every
    root-to-leaf path as its own isolated sequence (attention and GDN,
    literal mode).  The other workloads: seeded leaf paths, extrapolated."""
    import oracle
    from workloads import make_config
    from workloads.tensors import draw_inputs

    if index in (2, 3, 4):
        return cpu_baseline_sampled(index, {2: 4, 3: 1, 4: 4}[index])
    cfg, tree = make_config(index, n_requests=n_req)
    inp = draw_inputs(tree, cfg.shapes, cfg.seed, cfg.dtype, cfg.mu_a)
    ts, par, fkk, cl = tree.arrays()
    args = {n: inp.f64(n) for n in inp.raw}
    t0 = time.perf_counter()
    oracle.attention(ts, par, fkk, cl, inp.hist_off, args["aq"], args["ak"], args["av"], None, None,
                     cfg.shapes.d ** -0.5, mode=0)
    oracle.gdn(ts, par, fkk, cl, args["gq"], args["gk"], args["gv"], args["ga"], args["gb"], mode=0)
    dt = time.perf_counter() - t0
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    bt = tree.branch_tokens()
    return {"value": bt / dt, "unit": "branch tokens/s", "cores": cores, "kind": "oracle", **host_cpu(),
            "extrapolated": False,
            "sample": f"first {n_req} request(s) of the workload ({tree.T} stream tokens, {bt} branch "
                      f"tokens, {len(tree.leaves())} leaf paths), fp64 literal isolated-path "
                      f"attention + GDN, {dt:.1f} s"}


def path_work(tree, leaf):
    """(live rows L, cached history rows H) of a leaf's isolated path: the
    literal oracle evaluates each live row r over its H + r + 1 keys
    (L H + L (L + 1) / 2 attention pairs) and steps the recurrence over the L
    live rows from the history's saved state."""
    L, H, j = tree.segs[leaf].length, 0, leaf
    while tree.segs[j].parent >= 0:
        p = tree.segs[j].parent
        if tree.segs[p].cached:
            H += tree.segs[j].fork
        else:
            L += tree.segs[j].fork
        j = p
    return L, H


def cpu_baseline_sampled(index: int, n_paths: int):
    """The fp64 oracle on the long-path workloads (a literal run of every leaf
    path would take from an hour to days): ``n_paths`` seeded leaf paths, each
    run alone in literal mode -- its whole isolated sequence, history keys
    included, with one attention q head and one GDN v-head timed -- scaled to
    every head and every leaf path (attention by the paths' visible pairs,
    GDN by their live rows).  On the resume workload the sampled leaves come
    from one seeded request, whose history state the oracle makes first,
    untimed, as the GPU's checkpoint pass does.  The figure is extrapolated
    and says so."""
    import oracle
    from workloads import make_config, subtree_path
    from workloads.tensors import draw_inputs

    cfg, tree = make_config(index)
    sh = cfg.shapes
    leaves = tree.leaves()
    rng = np.random.default_rng(index)
    if index == 4:
        req = int(rng.integers(tree.n_requests))
        pool = [i for i, x in enumerate(leaves) if tree.segs[x].request == req]
    else:
        pool = list(range(len(leaves)))
    pick = rng.choice(pool, size=min(n_paths, len(pool)), replace=False)
    work = np.array([path_work(tree, x) for x in leaves], np.float64)
    pairs = work[:, 0] * work[:, 1] + work[:, 0] * (work[:, 0] + 1) / 2
    a_sel = (np.arange(sh.Hq) == 0).astype(np.uint8)
    g_sel = (np.arange(sh.Hv) == 0).astype(np.uint8)
    cache = {}
    t_attn = t_gdn = 0.0
    for li in pick:
        leaf = int(leaves[li])
        sub, _ = subtree_path(tree, leaf)
        sub.flatten()
        inp = draw_inputs(sub, sh, cfg.seed, cfg.dtype, cfg.mu_a, request_streams=[tree.segs[leaf].request],
                          cache=cache)
        ts, par, fkk, cl = sub.arrays()
        args = {n: inp.f64(n) for n in inp.raw}
        st_in, ssi = None, None
        hist = [i for i, s in enumerate(sub.segs) if s.cached]
        if hist:   # the history's final state, made untimed (the GPU's checkpoint pass)
            h = sub.segs[hist[0]].length
            z = np.zeros(1, np.int32)
            _, st_in, _ = oracle.gdn(np.zeros(h, np.int32), z - 1, z, z, inp.f64("gq", True), inp.f64("gk", True),
                                     inp.f64("gv", True), inp.f64("ga", True), inp.f64("gb", True),
                                     seg_state_out=np.zeros(1, np.int32), n_state_out=1, mode=1, head_sel=g_sel)
            ssi = np.full(sub.S, -1, np.int32)
            ssi[hist[0]] = 0
        t0 = time.perf_counter()
        oracle.attention(ts, par, fkk, cl, inp.hist_off, args["aq"], args["ak"], args["av"], inp.f64("ak", True),
                         inp.f64("av", True), sh.d ** -0.5, mode=0, head_sel=a_sel)
        t1 = time.perf_counter()
        oracle.gdn(ts, par, fkk, cl, args["gq"], args["gk"], args["gv"], args["ga"], args["gb"], state_in=st_in,
                   seg_state_in=ssi, mode=0, head_sel=g_sel)
        t2 = time.perf_counter()
        t_attn += (t1 - t0) * sh.Hq
        t_gdn += (t2 - t1) * sh.Hv
    total = t_attn * pairs.sum() / pairs[pick].sum() + t_gdn * work[:, 0].sum() / work[pick, 0].sum()
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    bt = tree.branch_tokens()
    where = f" of request {req}" if index == 4 else ""
    return {"value": bt / total, "unit": "branch tokens/s", "cores": cores, "kind": "oracle", **host_cpu(),
            "extrapolated": True,
            "sample": f"{len(pick)} of {len(leaves)} leaf paths (seeded{where}), each alone in fp64 literal mode, "
                      f"one attention q head and one GDN v-head timed "
                      f"({(t_attn / sh.Hq + t_gdn / sh.Hv):.1f} s), scaled to all {sh.Hq} q / {sh.Hv} v heads "
                      f"and to every leaf path (by visible pairs for attention, by live rows for GDN): "
                      f"{total:.0f} s for the whole workload"}


def make_workload(index: int):
    if index == 4:
        wl = ResumeWorkload()
        wl.checkpoint()
        return wl
    return Workload(index)


def measure(index: int, args, next_rows: bool):
    """Step one workload: eager steps with HIP events at the phase boundaries
    (the per-phase times and the kernels' durations for the rooflines), then
    the step recorded as a HIP graph and replayed (the headline timing).
    Returns the workload's fields of the JSON line."""
    import torch

    wl = make_workload(index)
    tree, sh = wl.tree, wl.sh
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()
    assert wl.fk.fk_read_status(wl.ws) == 0, "tree build reported an error"
    # eager pass: per-phase times with HIP events on the launch stream (these
    # give the phases and the kernels' durations for the rooflines)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        wl.step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    phase = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in evs])  # ms
    ms_eager = wall * 1e3 / args.steps
    ms_step, mode = ms_eager, "eager launches"
    dist, forms, n_warm = None, {}, None
    if not args.eager:
        # the same step recorded once as a HIP graph and replayed: the
        # headline timing (no launch gaps between the step's kernels).  Both
        # forms of the step are recorded -- serial, and the GDN phase on a
        # second stream beside the append and the attention -- and the one
        # whose warm replays are faster is timed: the overlap pays where
        # the GDN phase is comparable to the attention (the mixture) and
        # costs where a long attention launch shares the chip with it.
        def warm(g):
            # untimed replays: at least `warmup`, and at least 30 ms of them
            # (the first ~20 replays of the mixture run ~6% slower while the
            # clocks settle)
            n, tw = 0, time.perf_counter()
            while n < args.warmup or time.perf_counter() - tw < 0.03:
                g.replay()
                n += 1
                if n % 8 == 0:
                    torch.cuda.synchronize()
            torch.cuda.synchronize()
            return n

        def replay_ms(g, n):
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
            for e in ev:
                e[0].record()
                g.replay()
                e[1].record()
            torch.cuda.synchronize()
            return np.array([e[0].elapsed_time(e[1]) for e in ev])

        n_warm = 0
        for name, fn in (("serial", wl.step), ("GDN phase on a second stream", wl.step_overlapped)):
            g = wl.fk.StepGraph(fn, warmup=1)
            n_warm += warm(g)
            forms[name] = (float(np.median(replay_ms(g, 5))), g)
        form = min(forms, key=lambda k: forms[k][0])
        graph = forms[form][1]
        n_warm += warm(graph)
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
        mode = f"HIP graph replay ({form})"
        assert wl.fk.fk_read_status(wl.ws) == 0, "tree build reported an error"
        # per-replay distribution (HIP events), warm and with the caches
        # flushed before each step (a 512 MiB write evicts L2 and MALL)
        warm_ms = replay_ms(graph, args.steps)
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        cold = []
        for _ in range(min(args.steps, 10)):
            flush.zero_()
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record()
            graph.replay()
            e[1].record()
            torch.cuda.synchronize()
            cold.append(e[0].elapsed_time(e[1]))
        del flush
        dist = {"warm_p10": float(np.percentile(warm_ms, 10)), "warm_p50": float(np.percentile(warm_ms, 50)),
                "warm_p90": float(np.percentile(warm_ms, 90)), "cold_p50": float(np.median(cold)),
                "cold_flush_bytes": 512 << 20}
        forms = {k: v[0] for k, v in forms.items()}
        del graph, g
    resume = index == 4
    elem = 2 if wl.cfg.dtype == "bf16" else 4
    attn_ms = float(phase[:, 2].mean())
    nvis = visible_pairs(tree)
    flops = 4.0 * sh.d * sh.Hq * nvis
    achieved = flops / (attn_ms * 1e-3) / 1e12
    bt = tree.branch_tokens()
    kv_ms = float(phase[:, 1].mean())
    kvb = kv_bytes(tree, sh, elem)
    out = {
        "value": bt / (ms_step * 1e-3),
        "unit": "branch tokens/s",
        "ms_per_step": ms_step,
        "dtype": wl.cfg.dtype,
        "config": {"workload": wl.cfg.name, "index": index, "requests": tree.n_requests,
                   "stream_tokens": tree.T, "branch_tokens": bt, "segments": tree.S,
                   "leaves": len(tree.leaves()), "attn_heads": [sh.Hq, sh.Hkv, sh.d],
                   "gdn_heads": [sh.Hk, sh.Hv, sh.dk, sh.dv]},
        "execution": mode,
        "graph_bucket": {"stream_tokens": wl.bucket.T, "segment_slots": wl.bucket.S,
                         "levels": wl.bucket.max_depth, "level_cap": wl.bucket.level_cap,
                         "fork_cap": wl.bucket.fork_cap},
        "graph_warmup_replays": n_warm,
        "graph_forms_ms": forms or None,
        "step_ms_distribution": dist,
        "stream_tokens_per_s": tree.T / (ms_step * 1e-3),
        "path_equivalent_tokens_per_s": path_tokens(tree) / (ms_step * 1e-3),
        "ms_per_step_eager": ms_eager,
        "phases_ms": {("resume+tree_build" if resume else "tree_build"): float(phase[:, 0].mean()),
                      "kv_append": kv_ms, "fork_attention": attn_ms,
                      ("gdn+checkpoint_save" if resume else "gdn"): float(phase[:, 3].mean())},
        "roofline": {"kernel": "fork attention (bf16 MFMA)", "bound": "mfma", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic("attention", index), "ms": attn_ms,
                     "algorithmic_flops": flops, "visible_pairs_per_head": nvis},
        "kv_roofline": {"kernel": "paged K/V append (bf16)", "bound": "hbm", "ms": kv_ms,
                        "achieved": kvb / (kv_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": kvb / (kv_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "traffic": measured_traffic("kv_append", index), "algorithmic_bytes": kvb},
    }
    if getattr(wl, "gdn_ok", True):
        gdn_ms = float(phase[:, 3].mean())
        nbytes = gdn_bytes(tree, sh, elem, resumed_save=resume)
        n_forks, children, _ = gdn_forks(tree)
        gbs = nbytes / (gdn_ms * 1e-3) / 1e9
        out["gdn_roofline"] = {"kernels": "GDN prep + one chunk walk per tree level (bf16 MFMA)"
                                          + (" + checkpoint save" if resume else ""),
                               "bound": "hbm", "ms": gdn_ms, "achieved": gbs, "peak": PEAK_HBM_GBS,
                               "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS, "algorithmic_bytes": nbytes,
                               "traffic": measured_traffic("gdn", index), "fork_points": n_forks,
                               "bytes_if_each_child_copied_its_state":
                                   nbytes + (children - n_forks) * sh.Hv * sh.dv * sh.dk * 4}
    else:
        out["incomplete"] = "gdn_fork_forward does not support this dtype: the step lacks GDN"
    if next_rows:
        out["next_rows"] = {"conv": measure_conv(wl, args.steps),
                            "window_attention": measure_rule(wl, args.steps, 1, 1024),
                            "two_way_attention": measure_rule(wl, args.steps, 2),
                            "readout": measure_readout(wl, args.steps),
                            "projection": measure_proj(wl, args.steps)}
    del wl
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py runs on one GPU; runs on several GPUs are not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
    also = [int(x) for x in args.also.split(",") if x.strip() and int(x) != args.config]
    print(f"[bench] workload {args.config}", file=sys.stderr, flush=True)
    head = measure(args.config, args, next_rows=not args.no_next_rows)
    line = {"metric": METRIC, "value": head.pop("value"), "unit": head.pop("unit"), "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": head.pop("ms_per_step"),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": head.pop("dtype"),
            "data": "synthetic", "config": head.pop("config")}
    line.update(head)
    others = {}
    for i in also:
        print(f"[bench] workload {i}", file=sys.stderr, flush=True)
        others[str(i)] = measure(i, args, next_rows=False)
    if others:
        line["configs"] = others
    line["measured_peaks"] = measured_peaks()
    if not args.no_cpu_baseline:
        print("[bench] cpu baselines", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args.config, args.cpu_requests)
        for i, o in others.items():
            o["cpu_baseline"] = cpu_baseline(int(i), args.cpu_requests)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
