"""GPU parity of the float32 path against the fp64 oracle (max-abs 1e-4),
the builder's canonical indexing (bit-exact), device-side validation, and
run-twice determinism.  Calls go through the C-ABI binding."""
import numpy as np
import pytest
import torch

import gated_deltanet_amd as fk
import oracle
from tests.harness import GpuRound, oracle_attention, oracle_gdn, to_f64
from tests.malformed import CASES, arrays
from workloads import make_config, random_tree
from workloads.tensors import Shapes, draw_inputs
from workloads.configs import WORKLOADS

pytestmark = pytest.mark.gpu
TOL = 1e-4


def _cfg0():
    cfg, t = make_config(0)
    return draw_inputs(t, cfg.shapes, cfg.seed, cfg.dtype, cfg.mu_a)


def _random_inputs(seed, shapes=Shapes(4, 2, 64, 2, 4, 32, 32), **kw):
    rng = np.random.default_rng(seed)
    t = random_tree(rng, p_cached_root=0.4, p_internal_fork=0.4, **kw)
    order = None
    if seed % 2:
        live = [i for i, s in enumerate(t.segs) if not s.cached]
        order = list(rng.permutation(live))
    t.flatten(order)
    return draw_inputs(t, shapes, 500 + seed, "f32"), rng


@pytest.mark.parametrize("which", [0, 1, 2, 3, 4])
def test_positions_match_oracle(which):
    print(f"[positions] config {which}", flush=True)
    cfg, t = make_config(which)
    ts, par, fkk, cl = t.arrays()
    ssi = np.where(cl > 0, np.cumsum(cl > 0) - 1, -1)
    plan = fk.plan_round(ts, par, fkk, cl, cached_pages={s: [0] * (-(-int(cl[s]) // 16)) for s in range(t.S) if cl[s]},
                         seg_state_in=ssi, n_state_in=int((cl > 0).sum()))
    ws = fk.alloc_workspace(plan.meta)
    fk.fk_tree_build(plan.meta, ws)
    assert fk.fk_read_status(ws) == 0
    pos = fk.fk_token_positions(plan.meta, ws).cpu().numpy()
    np.testing.assert_array_equal(pos, oracle.index(ts, par, fkk, cl)["tok_pos"])


def test_positions_random_trees():
    for seed in range(12):
        inp, _ = _random_inputs(seed)
        r = GpuRound(inp).build()
        assert r.status() == 0
        pos = fk.fk_token_positions(r.meta, r.ws).cpu().numpy()
        np.testing.assert_array_equal(pos, oracle.index(*inp.tree.arrays())["tok_pos"])


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_device_validation_matches_host(case):
    ts, par, fkk, cl, kind = arrays(case)
    S = len(par)
    off = np.arange(0, 8 * (S + 1), 8)
    pages = np.arange(8 * S)
    ssi = np.where(cl > 0, 0, -1)
    host = fk.fk_tree_validate_host(ts, par, fkk, cl, off, pages, 8 * S, ssi, None, 1, 0)
    meta = fk.make_tree_meta(ts, par, fkk, cl, off, pages, 8 * S, ssi, None, 1, 0)
    ws = fk.alloc_workspace(meta)
    fk.fk_tree_build(meta, ws)
    dev = fk.fk_read_status(ws)
    assert host != 0 and dev == host, (host, dev)


def test_attention_f32_config0():
    inp = _cfg0()
    r = GpuRound(inp).build()
    o = to_f64(r.attention())
    assert r.status() == 0
    ref = oracle_attention(inp)
    err = np.abs(o - ref).max()
    print(f"[attn f32 cfg0] max-abs {err:.3e}", flush=True)
    assert err <= TOL


@pytest.mark.parametrize("d", [32, 64, 128])
def test_attention_f32_random_trees(d):
    for seed in range(8):
        inp, _ = _random_inputs(seed, Shapes(6, 2, d, 2, 4, 32, 32))
        r = GpuRound(inp).build()
        o = to_f64(r.attention())
        assert r.status() == 0
        ref = oracle_attention(inp)
        assert np.abs(o - ref).max() <= TOL, (seed, np.abs(o - ref).max())


def test_gdn_f32_config0():
    inp = _cfg0()
    r = GpuRound(inp).build()
    o = to_f64(r.gdn())
    assert r.status() == 0
    ref, st = oracle_gdn(inp)
    err = np.abs(o - ref).max()
    serr = np.abs(to_f64(r.state_out)[: len(st)] - st).max()
    print(f"[gdn f32 cfg0] max-abs out {err:.3e} state {serr:.3e}", flush=True)
    assert err <= TOL and serr <= TOL


@pytest.mark.parametrize("dk,dv", [(32, 32), (64, 16), (16, 128), (128, 128)])
def test_gdn_f32_random_trees(dk, dv):
    for seed in range(8):
        inp, rng = _random_inputs(seed, Shapes(2, 1, 16, 2, 4, dk, dv))
        n_in = sum(s.cached for s in inp.tree.segs)
        st_in = rng.standard_normal((n_in, 4, dv, dk)).astype(np.float32) * 0.3 if n_in else None
        r = GpuRound(inp, state_in_np=st_in).build()
        o = to_f64(r.gdn())
        assert r.status() == 0
        ref, st = oracle_gdn(inp, state_in=st_in)
        assert np.abs(o - ref).max() <= TOL, (seed, np.abs(o - ref).max())
        assert np.abs(to_f64(r.state_out)[: len(st)] - st).max() <= TOL


def test_f32_run_twice_bitwise():
    inp, _ = _random_inputs(3)
    r = GpuRound(inp).build()
    a1, g1 = r.attention().clone(), r.gdn().clone()
    a2, g2 = r.attention().clone(), r.gdn().clone()
    assert torch.equal(a1, a2) and torch.equal(g1, g2)
