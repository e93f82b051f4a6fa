#!/usr/bin/env python3
"""Benchmark one forked pass of the hot path on one MI355X.

A step is one pass over one round of synthetic decision requests: the
tree-metadata build, the paged K/V append, ForkAttention over the round
(GQA softmax attention, every branch seeing only its ancestry), and the
forked Gated DeltaNet layer (trunk once, children from the fork-point state
by index); for the resume workload also the checkpoint resume and save.

Default workload: the 16-request decision mixture (trunks ~U[512, 2048],
4-8 branches of ~U[16, 48] tokens, bf16, attention 16q/2kv heads d128, GDN
16 heads 128x128).  Prints ONE JSON line with the throughput in branch
tokens/s, the dominant kernel's roofline and the fp64 CPU oracle timed on
a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--config 1]
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
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=1, help="workload index (0-4)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-requests", type=int, default=16,
                    help="requests of the workload in the CPU oracle sample")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run one plain copy of 256 MiB (gdn_checkpoint_save) before timing, so a "
                         "counter run can scale FETCH_SIZE / WRITE_SIZE to bytes")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_mixture_traffic.txt")
ATTN_SRC = os.path.join(ROOT, "gated_deltanet_amd", "csrc", "attn_bf16.hip")


def kernel_hash(path: str) -> str:
    import hashlib
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def measured_traffic(config: int):
    """HBM bytes per attention launch from the committed counter summary, or
    None when it is missing, for another workload, or the kernel changed."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        parts = line.split()
        if len(parts) == 2 and not line.startswith("#"):
            kv[parts[0]] = parts[1]
    if kv.get("kernel_sha256_16") != kernel_hash(ATTN_SRC) or kv.get("config") != str(config):
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


class Workload:
    """A config's round resident on the GPU, ready to step."""

    def __init__(self, index: int, device="cuda"):
        import torch

        import gated_deltanet_amd as fk
        from workloads import make_config
        from workloads.tensors import draw_inputs

        self.torch, self.fk = torch, fk
        cfg, tree = make_config(index)
        if any(s.cached for s in tree.segs):
            raise SystemExit("the resume workload needs its history pass; not wired into the bench yet")
        self.cfg, self.tree = cfg, tree
        inp = draw_inputs(tree, cfg.shapes, cfg.seed, cfg.dtype, cfg.mu_a)
        sh = cfg.shapes
        self.sh = sh
        dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

        def dev(name):
            x = torch.from_numpy(np.ascontiguousarray(inp.raw[name]))
            if x.dtype == torch.int16 or inp.raw[name].dtype == np.uint16:
                x = x.view(torch.bfloat16)
            return x.to(device)

        self.x = {n: dev(n) for n in inp.raw}
        del inp
        ts, par, fkk, cl = tree.arrays()
        sso = np.full(tree.S, -1, np.int32)
        self.plan = fk.plan_round(ts, par, fkk, cl, seg_state_out=sso, n_state_out=0, device=device)
        self.meta = self.plan.meta
        self.ws = fk.alloc_workspace(self.meta, sh.Hv, sh.dk, sh.dv, device=device)
        n_pages = self.plan.n_pages
        self.k_pool = torch.zeros((n_pages, sh.Hkv, 16, sh.d), dtype=dt, device=device)
        self.v_pool = torch.zeros((n_pages, sh.Hkv, sh.d, 16), dtype=dt, device=device)
        self.attn_out = torch.empty_like(self.x["aq"])
        self.gdn_out = torch.empty_like(self.x["gv"])
        self.scale = sh.d ** -0.5
        self.gdn_ok = True

    def step(self, ev=None):
        fk, x = self.fk, self.x
        if ev:
            ev[0].record()
        fk.fk_tree_build(self.meta, self.ws)
        if ev:
            ev[1].record()
        fk.kv_append(self.meta, x["ak"], x["av"], self.k_pool, self.v_pool, self.ws)
        if ev:
            ev[2].record()
        fk.fork_attn_forward(self.meta, x["aq"], None, None, self.k_pool, self.v_pool, self.ws,
                             scale=self.scale, out=self.attn_out)
        if ev:
            ev[3].record()
        if self.gdn_ok:
            try:
                fk.gdn_fork_forward(self.meta, x["gq"], x["gk"], x["gv"], x["ga"], x["gb"], self.ws,
                                    out=self.gdn_out)
            except fk._lib.FkError as e:   # reported in the JSON line, never silently
                if e.name != "FK_E_UNSUPPORTED":
                    raise
                self.gdn_ok = False
        if ev:
            ev[4].record()


def cpu_baseline(index: int, n_req: int):
    """The fp64 oracle, as it stands, on the first ``n_req`` requests of the
    same workload: every root-to-leaf path as its own isolated sequence
    (attention and GDN, literal mode).  Returns branch tokens/s."""
    import oracle
    from workloads import make_config
    from workloads.tensors import draw_inputs

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
    return {"value": bt / dt, "unit": "branch tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"first {n_req} request(s) of the workload ({tree.T} stream tokens, {bt} branch "
                      f"tokens, {len(tree.leaves())} leaf paths), fp64 literal isolated-path "
                      f"attention + GDN, {dt:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; multi-GPU runs are not part of it",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    if args.calibrate_copy:
        calibrate_copy()
    wl = Workload(args.config)
    tree, sh = wl.tree, wl.sh
    for _ in range(args.warmup):
        wl.step()
    torch.cuda.synchronize()
    assert wl.fk.fk_read_status(wl.ws) == 0, "tree build reported an error"
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        wl.step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    phase = np.array([[e[j].elapsed_time(e[j + 1]) for j in range(4)] for e in evs])  # ms
    ms_step = wall * 1e3 / args.steps
    attn_ms = float(phase[:, 2].mean())
    nvis = visible_pairs(tree)
    flops = 4.0 * sh.d * sh.Hq * nvis
    achieved = flops / (attn_ms * 1e-3) / 1e12
    bt = tree.branch_tokens()
    line = {
        "metric": METRIC,
        "value": bt / (ms_step * 1e-3),
        "unit": "branch tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.cfg.dtype,
        "data": "synthetic",
        "config": {"workload": wl.cfg.name, "index": args.config, "requests": tree.n_requests,
                   "stream_tokens": tree.T, "branch_tokens": bt, "segments": tree.S,
                   "attn_heads": [sh.Hq, sh.Hkv, sh.d], "gdn_heads": [sh.Hk, sh.Hv, sh.dk, sh.dv]},
        "phases_ms": {"tree_build": float(phase[:, 0].mean()), "kv_append": float(phase[:, 1].mean()),
                      "fork_attention": attn_ms, "gdn": float(phase[:, 3].mean())},
        "roofline": {"kernel": "fork attention (bf16 MFMA)", "bound": "mfma", "achieved": achieved,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                     "traffic": measured_traffic(args.config), "algorithmic_flops": flops,
                     "visible_pairs_per_head": nvis},
    }
    if not wl.gdn_ok:
        line["incomplete"] = "gdn_fork_forward unsupported for this dtype in this build: step lacks GDN"
        line["phases_ms"]["gdn"] = None
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.config, args.cpu_requests)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
