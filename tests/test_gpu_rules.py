"""ForkAttention under the other visibility rules of Flide section 3.2.1
(sliding window: t_x - t_y < W; two-way: the whole own segment, Flide
appendix H) against the fp64 oracle: fp32 max-abs 1e-4; bf16 max-abs 2e-2
and mean-abs 2e-3; a window wider than every path equals the causal rule bit
for bit; and batch invariance -- a leaf alone gives the same bits as in the
round."""
import numpy as np
import pytest

import gated_deltanet_amd as fk
from gated_deltanet_amd._lib import FK_RULE_CAUSAL, FK_RULE_TWO_WAY, FK_RULE_WINDOW
from tests.harness import GpuRound, config_inputs, oracle_attention, to_f64
from workloads import random_tree, subtree_path
from workloads.tensors import Shapes, draw_inputs

pytestmark = pytest.mark.gpu
BF16 = (2e-2, 2e-3)
F32 = (1e-4, 1e-4)
SH_BF16 = Shapes(16, 2, 128, 2, 4, 128, 128)
SH_F32 = Shapes(4, 2, 64, 2, 4, 32, 32)

CASES = [(FK_RULE_WINDOW, 1), (FK_RULE_WINDOW, 7), (FK_RULE_WINDOW, 64), (FK_RULE_WINDOW, 100),
         (FK_RULE_WINDOW, 333), (FK_RULE_TWO_WAY, 0)]


def _tree(seed, max_len=150):
    rng = np.random.default_rng(5100 + seed)
    t = random_tree(rng, p_cached_root=0.4, p_internal_fork=0.4, max_len=max_len, max_cached=200)
    if seed % 2:
        live = [i for i, s in enumerate(t.segs) if not s.cached]
        t.flatten(list(rng.permutation(live)))
    else:
        t.flatten()
    return t


def _err(o, ref):
    assert np.isfinite(o).all()
    d = np.abs(o - ref)
    return d.max(), d.mean()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rules_random_trees(dtype):
    sh, (mx_tol, mean_tol) = (SH_BF16, BF16) if dtype == "bf16" else (SH_F32, F32)
    for seed in range(6):
        t = _tree(seed)
        inp = draw_inputs(t, sh, 61 + seed, dtype)
        r = GpuRound(inp).build()
        for rule, W in CASES:
            print(f"[rules {dtype}] seed {seed} T={t.T} rule {rule} W={W}", flush=True)
            o = to_f64(r.attention(rule=rule, window=W))
            assert r.status() == 0
            mx, mean = _err(o, oracle_attention(inp, rule=rule, window=W))
            print(f"  max {mx:.2e} mean {mean:.2e}", flush=True)
            assert mx <= mx_tol and mean <= mean_tol, (seed, rule, W, mx, mean)


def test_window_wider_than_paths_is_causal():
    t = _tree(11)
    inp = draw_inputs(t, SH_BF16, 5, "bf16")
    r = GpuRound(inp).build()
    causal = to_f64(r.attention())
    wide = to_f64(r.attention(rule=FK_RULE_WINDOW, window=1 << 20))
    explicit = to_f64(r.attention(rule=FK_RULE_CAUSAL))
    assert np.array_equal(causal, wide) and np.array_equal(causal, explicit)


@pytest.mark.parametrize("rule,W", [(FK_RULE_WINDOW, 100), (FK_RULE_TWO_WAY, 0)])
def test_rules_batch_invariance(rule, W):
    t = _tree(12, max_len=120)
    inp = draw_inputs(t, SH_BF16, 8, "bf16")
    r = GpuRound(inp).build()
    o = to_f64(r.attention(rule=rule, window=W))
    starts = {}
    for x, s in enumerate(t.tok_seg):
        starts.setdefault(int(s), x)
    leaves = [i for i, s in enumerate(t.segs) if not s.cached and not t.children(i)]
    for leaf in leaves:
        sub, chain = subtree_path(t, leaf)
        sub.flatten()
        ia = draw_inputs(sub, SH_BF16, 8, "bf16", request_streams=[t.segs[leaf].request])
        ra = GpuRound(ia).build()
        oa = to_f64(ra.attention(rule=rule, window=W))
        sub_starts = {}
        for x, s in enumerate(sub.tok_seg):
            sub_starts.setdefault(int(s), x)
        for new, old in enumerate(chain):
            if t.segs[old].cached:
                continue
            n = t.segs[old].length
            assert np.array_equal(oa[sub_starts[new]: sub_starts[new] + n], o[starts[old]: starts[old] + n]), leaf


@pytest.mark.parametrize("which,rule,W", [(1, FK_RULE_WINDOW, 512), (1, FK_RULE_TWO_WAY, 0),
                                          (3, FK_RULE_WINDOW, 4096)])
def test_rules_configs_sampled(which, rule, W):
    """Full-size workloads in the bench's launch configuration, on sampled
    rows (each segment's first, last and one random row) and a quarter of the
    heads."""
    cfg, inp = config_inputs(which)
    t = inp.tree
    print(f"[rules config {which}] rule {rule} W={W} T={t.T}", flush=True)
    r = GpuRound(inp).build()
    o = to_f64(r.attention(rule=rule, window=W))
    assert r.status() == 0
    rng = np.random.default_rng(which)
    sel = np.zeros(t.T, bool)
    starts = {}
    for x, s in enumerate(t.tok_seg):
        starts.setdefault(int(s), x)
    for s, st in starts.items():
        L = t.segs[s].length
        for i in {0, L - 1, int(rng.integers(L))}:
            sel[st + i] = True
    hs = np.arange(0, cfg.shapes.Hq, 4)
    hsel = np.zeros(cfg.shapes.Hq, np.uint8)
    hsel[hs] = 1
    ref = oracle_attention(inp, tok_sel=sel.astype(np.uint8), rule=rule, window=W, head_sel=hsel)
    mx, mean = _err(o[sel][:, hs], ref[sel][:, hs])
    print(f"  max {mx:.2e} mean {mean:.2e}", flush=True)
    assert mx <= BF16[0] and mean <= BF16[1]
