"""Selective readout (fork_attn_readout, Flide section 3.3.3): attention at the
rows of an index buffer only.  Each entry's output must have the same bits as
that token's row of the full launch under the same rule, match the fp64
oracle on those rows (fp32 max-abs 1e-4; bf16 max-abs 2e-2, mean-abs 2e-3),
and unused entries (-1) must leave their output rows untouched."""
import numpy as np
import pytest
import torch

import gated_deltanet_amd as fk
from gated_deltanet_amd._lib import FK_RULE_CAUSAL, FK_RULE_TWO_WAY, FK_RULE_WINDOW
from tests.harness import GpuRound, config_inputs, oracle_attention, to_f64
from workloads import random_tree
from workloads.tensors import Shapes, draw_inputs

pytestmark = pytest.mark.gpu
TOL = {"bf16": (2e-2, 2e-3), "f32": (1e-4, 1e-4)}
SH = {"bf16": Shapes(16, 2, 128, 2, 4, 128, 128), "f32": Shapes(4, 2, 64, 2, 4, 32, 32)}


def _row_buffer(tree, rng, extra=4):
    """Every leaf's last token, a few random tokens, one duplicate and unused
    (-1) entries, shuffled -- a fixed-size buffer as a graph would hold."""
    starts = {}
    for x, s in enumerate(tree.tok_seg):
        starts.setdefault(int(s), x)
    rows = [starts[i] + tree.segs[i].length - 1 for i in range(tree.S)
            if not tree.segs[i].cached and not tree.children(i)]
    rows += [int(x) for x in rng.integers(0, tree.T, extra)]
    rows += [rows[0], -1, -1]
    rows = np.array(rows, np.int32)
    rng.shuffle(rows)
    return rows


def _readout(r, rows, rule, W):
    q = r.x["aq"]
    rows_t = torch.from_numpy(rows).cuda()
    idx = torch.from_numpy(np.where(rows >= 0, rows, 0)).long().cuda()
    q_rows = q[idx].contiguous()
    q_rows[torch.from_numpy(rows < 0).cuda()] = 0
    out = torch.full_like(q_rows, float("nan"))
    fk.fork_attn_readout(r.meta, q_rows, rows_t, r.k_pool, r.v_pool, r.ws, rule=rule, window=W, out=out)
    return to_f64(out)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rule,W", [(FK_RULE_CAUSAL, 0), (FK_RULE_WINDOW, 37), (FK_RULE_TWO_WAY, 0)])
def test_readout_random_trees(dtype, rule, W):
    for seed in range(5):
        rng = np.random.default_rng(6200 + seed)
        t = random_tree(rng, p_cached_root=0.4, p_internal_fork=0.4, max_len=120)
        if seed % 2:
            live = [i for i, s in enumerate(t.segs) if not s.cached]
            t.flatten(list(rng.permutation(live)))
        else:
            t.flatten()
        inp = draw_inputs(t, SH[dtype], 300 + seed, dtype)
        print(f"[readout {dtype}] seed {seed} rule {rule} T={t.T}", flush=True)
        r = GpuRound(inp).build()
        full = to_f64(r.attention(rule=rule, window=W))     # also pages this round's K/V
        rows = _row_buffer(t, rng)
        o = _readout(r, rows, rule, W)
        assert r.status() == 0
        used = rows >= 0
        assert np.isnan(o[~used]).all(), "unused entries must stay untouched"
        assert np.array_equal(o[used], full[rows[used]]), "readout differs from the full launch"
        sel = np.zeros(t.T, np.uint8)
        sel[rows[used]] = 1
        ref = oracle_attention(inp, tok_sel=sel, rule=rule, window=W)
        d = np.abs(o[used] - ref[rows[used]])
        mx, mean = TOL[dtype]
        assert d.max() <= mx and d.mean() <= mean, (seed, d.max(), d.mean())


def test_readout_config3_leaves():
    """The 32k-trunk workload: the last token of each of the 64 questions,
    bit-identical to the full launch, and within the bf16 bar of the oracle
    on a quarter of the heads."""
    cfg, inp = config_inputs(3)
    t = inp.tree
    r = GpuRound(inp).build()
    full = to_f64(r.attention())
    rows = _row_buffer(t, np.random.default_rng(3), extra=0)
    o = _readout(r, rows, FK_RULE_CAUSAL, 0)
    used = rows >= 0
    assert np.array_equal(o[used], full[rows[used]])
    sel = np.zeros(t.T, np.uint8)
    sel[rows[used]] = 1
    hsel = np.zeros(cfg.shapes.Hq, np.uint8)
    hsel[::4] = 1
    ref = oracle_attention(inp, tok_sel=sel, head_sel=hsel)
    d = np.abs(o[used][:, ::4] - ref[rows[used]][:, ::4])
    assert d.max() <= 2e-2 and d.mean() <= 2e-3, (d.max(), d.mean())


@pytest.mark.parametrize("rule,W", [(FK_RULE_CAUSAL, 0), (FK_RULE_WINDOW, 45), (FK_RULE_TWO_WAY, 0)])
def test_readout_grouped_mixed_entries(rule, W):
    """A buffer large enough that entries are grouped 16 to a work-group, in
    shuffled order (each group mixes tokens of different segments, requests
    and depths, cached histories included): every entry still equals its row
    of the full launch bit for bit."""
    rng = np.random.default_rng(6400)
    t = random_tree(rng, n_requests=4, p_cached_root=0.4, p_internal_fork=0.4, max_len=100, max_depth=4).flatten()
    inp = draw_inputs(t, SH["bf16"], 77, "bf16")
    r = GpuRound(inp).build()
    full = to_f64(r.attention(rule=rule, window=W))
    rows = np.concatenate([rng.permutation(t.T) for _ in range(8)]).astype(np.int32)
    rows[rng.integers(0, len(rows), 50)] = -1
    print(f"[readout grouped] rule {rule} T={t.T} entries={len(rows)}", flush=True)
    o = _readout(r, rows, rule, W)
    assert r.status() == 0
    used = rows >= 0
    assert np.isnan(o[~used]).all()
    assert np.array_equal(o[used], full[rows[used]])


def test_readout_grouped_in_stream_order():
    """Entries in stream order, repeated, so that groups of 16 hold runs of one
    request and some straddle a request boundary (such a group's two parts are
    walked by two work-groups, one request's chains each): every entry equals
    its row of the full launch bit for bit, unused entries stay untouched."""
    rng = np.random.default_rng(6401)
    t = random_tree(rng, n_requests=6, p_cached_root=0.4, p_internal_fork=0.4, max_len=100, max_depth=4).flatten()
    inp = draw_inputs(t, SH["bf16"], 78, "bf16")
    r = GpuRound(inp).build()
    full = to_f64(r.attention())
    rows = np.concatenate([np.arange(t.T) for _ in range(8)]).astype(np.int32)
    rows[rng.integers(0, len(rows), 20)] = -1
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    group = min(16, len(rows) * SH["bf16"].Hkv // (3 * n_cu))
    print(f"[readout stream order] T={t.T} entries={len(rows)} group={group}", flush=True)
    assert group >= 8
    o = _readout(r, rows, FK_RULE_CAUSAL, 0)
    assert r.status() == 0
    used = rows >= 0
    assert np.isnan(o[~used]).all()
    assert np.array_equal(o[used], full[rows[used]])
