"""Parity at the workloads' full sizes, in the launch configuration the bench
times: the HIP path against the fp64 oracle on the same seeded inputs, per
output tensor (attention output, GDN output, GDN final states), max-abs and
mean-abs over every compared element, against the bf16 bar (2e-2 / 2e-3).

* decision-request mixture (16 requests): every element of every tensor --
  all rows, all heads, the final state of every live segment -- and every one
  of its leaves asked alone gives the mixture's bits (Flide section 3.5);
* agent fan-out (depth 3): every row on a quarter of the heads (two q heads
  of each kv group, every fourth v-head), with their final states;
* long shared context (32k trunks): a stratified sample -- the first and last
  row of every 16-token tile of every question, and the first and last row of
  every 64th trunk tile -- on every attention head; GDN on four v-heads over
  every token, with their final states.

The resume workload is checked at full size by ``test_gpu_resume.py``.
Positions of the paths follow Flide section 3.2 (Proposition 3.1: each branch
equals its isolated pass; the oracle runs those passes).
"""
import numpy as np
import pytest
import torch

from tests.harness import (GpuRound, config_inputs, oracle_attention, oracle_gdn, state_slots, stratified_rows,
                           to_f64)
from workloads import subtree_path
from workloads.tensors import draw_inputs

pytestmark = pytest.mark.gpu
MAX_ABS, MEAN_ABS = 2e-2, 2e-3


def _err(name, o, ref):
    assert np.isfinite(o).all(), name
    d = np.abs(o - ref)
    print(f"  {name}: max-abs {d.max():.3e} mean-abs {d.mean():.3e} over {d.size} elements", flush=True)
    return d.max(), d.mean()


def _check(name, o, ref):
    mx, mean = _err(name, o, ref)
    assert mx <= MAX_ABS and mean <= MEAN_ABS, (name, mx, mean)


def _starts(tree):
    st = {}
    for x, s in enumerate(tree.tok_seg):
        st.setdefault(int(s), x)
    return st


_RUNS = {}


def _run(i):
    """The workload's round through the C ABI, once per module: (config,
    inputs, round, attention output, GDN output) -- outputs as device tensors."""
    if i not in _RUNS:
        _RUNS.clear()
        cfg, inp = config_inputs(i)
        print(f"[config {i}] T={inp.tree.T} S={inp.tree.S}", flush=True)
        r = GpuRound(inp).build()
        a, g = r.attention(), r.gdn()
        torch.cuda.synchronize()
        assert r.status() == 0
        _RUNS[i] = (cfg, inp, r, a, g)
    return _RUNS[i]


def test_mixture_whole_tensors():
    cfg, inp, r, a, g = _run(1)
    _check("attention (all rows, all heads)", to_f64(a), oracle_attention(inp))
    ref, st = oracle_gdn(inp)
    _check("gdn (all rows, all heads)", to_f64(g), ref)
    _check("gdn final states (every live segment)", to_f64(r.state_out)[: len(st)], st)


def test_mixture_every_leaf_alone_bitwise():
    cfg, inp, r, a, g = _run(1)
    t = inp.tree
    st_mix = _starts(t)
    _, sso, _, _ = state_slots(t)
    cache = {}
    leaves = t.leaves()
    for n, leaf in enumerate(leaves):
        sub, chain = subtree_path(t, leaf)
        sub.flatten()
        ia = draw_inputs(sub, cfg.shapes, cfg.seed, cfg.dtype, cfg.mu_a, request_streams=[t.segs[leaf].request],
                         cache=cache)
        ra = GpuRound(ia).build()
        oa, og = ra.attention(), ra.gdn()
        assert ra.status() == 0
        _, sso_a, _, _ = state_slots(sub)
        st_a = _starts(sub)
        for new, old in enumerate(chain):
            L = t.segs[old].length
            x, y = st_a[new], st_mix[old]
            assert torch.equal(oa[x:x + L], a[y:y + L]), ("attention", leaf)
            assert torch.equal(og[x:x + L], g[y:y + L]), ("gdn", leaf)
            assert torch.equal(ra.state_out[sso_a[new]], r.state_out[sso[old]]), ("state", leaf)
        if n % 20 == 0:
            print(f"  leaf {n + 1}/{len(leaves)} alone: bit-identical", flush=True)
    print(f"  all {len(leaves)} leaves alone bit-identical to the mixture", flush=True)


def test_fanout_every_row_quarter_heads():
    cfg, inp, r, a, g = _run(2)
    sh = cfg.shapes
    hq = np.arange(0, sh.Hq, 4)       # two q heads of each kv group
    hv = np.arange(0, sh.Hv, 4)
    sel_q = np.zeros(sh.Hq, np.uint8)
    sel_q[hq] = 1
    sel_v = np.zeros(sh.Hv, np.uint8)
    sel_v[hv] = 1
    ref = oracle_attention(inp, head_sel=sel_q)
    _check(f"attention (all rows, q heads {list(hq)})", to_f64(a)[:, hq], ref[:, hq])
    gref, st = oracle_gdn(inp, head_sel=sel_v)
    _check(f"gdn (all rows, v heads {list(hv)})", to_f64(g)[:, hv], gref[:, hv])
    _check("gdn final states (those heads)", to_f64(r.state_out)[: len(st)][:, hv], st[:, hv])


def test_long_context_stratified():
    cfg, inp, r, a, g = _run(3)
    sh = cfg.shapes
    sel = stratified_rows(inp.tree)
    ref = oracle_attention(inp, tok_sel=sel.astype(np.uint8))
    _check(f"attention ({int(sel.sum())} stratified rows, all heads)", to_f64(a)[sel], ref[sel])
    hv = np.linspace(0, sh.Hv - 1, 4).astype(int)
    sel_v = np.zeros(sh.Hv, np.uint8)
    sel_v[hv] = 1
    gref, st = oracle_gdn(inp, head_sel=sel_v)
    _check(f"gdn (all rows, v heads {list(hv)})", to_f64(g)[:, hv], gref[:, hv])
    _check("gdn final states (those heads)", to_f64(r.state_out)[: len(st)][:, hv], st[:, hv])
