"""A round recorded once as a HIP graph and replayed (Flide section 3.3.2:
pre-recorded execution graphs, every round-dependent value in device
buffers).  Each replay -- with other eager work and synchronisations in
between -- must give the eager run's bits; after the inputs are refilled in
place, a replay must give the bits of an eager run on the new values."""
import numpy as np
import pytest
import torch

import gated_deltanet_amd as fk
from tests.harness import GpuRound
from workloads import random_tree
from workloads.tensors import Shapes, draw_inputs

pytestmark = pytest.mark.gpu
SH = Shapes(16, 2, 128, 2, 4, 128, 128)


def _round(seed):
    rng = np.random.default_rng(seed)
    t = random_tree(rng, n_requests=4, p_cached_root=0.3, p_internal_fork=0.4, max_len=120)
    t.flatten()
    inp = draw_inputs(t, SH, seed, "bf16")
    n_in = sum(s.cached for s in t.segs)
    st = (rng.standard_normal((n_in, SH.Hv, SH.dv, SH.dk)) * 0.2).astype(np.float32) if n_in else None
    return GpuRound(inp, state_in_np=st)


def _step(r, a_out, g_out):
    x = r.x
    fk.fk_tree_build(r.meta, r.ws)
    fk.kv_append(r.meta, x["ak"], x["av"], r.k_pool, r.v_pool, r.ws)
    fk.fork_attn_forward(r.meta, x["aq"], None, None, r.k_pool, r.v_pool, r.ws, out=a_out)
    fk.gdn_fork_forward(r.meta, x["gq"], x["gk"], x["gv"], x["ga"], x["gb"], r.ws, state_in=r.state_in,
                        state_out=r.state_out if r.n_out else None, out=g_out)


def test_graph_replay_bitwise():
    r = _round(31)
    print(f"[graph] T={r.inp.tree.T} S={r.inp.tree.S}", flush=True)
    a_out = torch.empty_like(r.x["aq"])
    g_out = torch.empty_like(r.x["gv"])
    _step(r, a_out, g_out)
    torch.cuda.synchronize()
    assert r.status() == 0
    a_ref, g_ref, s_ref = a_out.clone(), g_out.clone(), r.state_out.clone()
    graph = fk.StepGraph(lambda: _step(r, a_out, g_out))
    for rep in range(3):
        a_out.zero_()
        g_out.zero_()
        r.state_out.fill_(float("nan"))
        torch.cuda.synchronize()
        # unrelated eager work between replays
        z = torch.randn(512, 512, device="cuda")
        (z @ z).sum().item()
        graph.replay()
        torch.cuda.synchronize()
        assert r.status() == 0
        assert torch.equal(a_out, a_ref), rep
        assert torch.equal(g_out, g_ref), rep
        if r.n_out:
            assert torch.equal(r.state_out[: r.n_out], s_ref[: r.n_out]), rep
    # refill the inputs in place: the graph reads the live buffers
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    for name in ("aq", "ak", "av", "gv"):
        x = r.x[name]
        x.copy_(torch.randn(x.shape, generator=gen, device="cuda").to(x.dtype))
    graph.replay()
    torch.cuda.synchronize()
    a_g, g_g = a_out.clone(), g_out.clone()
    _step(r, a_out, g_out)
    torch.cuda.synchronize()
    assert torch.equal(a_g, a_out)
    assert torch.equal(g_g, g_out)
    assert not torch.equal(a_g, a_ref)


def test_graph_two_streams_bitwise():
    """The GDN calls read nothing the K/V append or the attention writes, so a
    round may run them on a second stream, forked after the build and joined
    at the end, inside one graph: every replay gives the serial run's bits."""
    r = _round(32)
    print(f"[graph two streams] T={r.inp.tree.T} S={r.inp.tree.S}", flush=True)
    a_out = torch.empty_like(r.x["aq"])
    g_out = torch.empty_like(r.x["gv"])
    _step(r, a_out, g_out)
    torch.cuda.synchronize()
    assert r.status() == 0
    a_ref, g_ref, s_ref = a_out.clone(), g_out.clone(), r.state_out.clone()
    side = torch.cuda.Stream()
    x = r.x

    def forked():
        fk.fk_tree_build(r.meta, r.ws)
        cur = torch.cuda.current_stream()
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            fk.gdn_fork_forward(r.meta, x["gq"], x["gk"], x["gv"], x["ga"], x["gb"], r.ws,
                                state_in=r.state_in, state_out=r.state_out if r.n_out else None, out=g_out)
        fk.kv_append(r.meta, x["ak"], x["av"], r.k_pool, r.v_pool, r.ws)
        fk.fork_attn_forward(r.meta, x["aq"], None, None, r.k_pool, r.v_pool, r.ws, out=a_out)
        cur.wait_stream(side)

    graph = fk.StepGraph(forked)
    for rep in range(3):
        a_out.zero_()
        g_out.zero_()
        r.state_out.fill_(float("nan"))
        torch.cuda.synchronize()
        z = torch.randn(512, 512, device="cuda")
        (z @ z).sum().item()
        graph.replay()
        torch.cuda.synchronize()
        assert r.status() == 0
        assert torch.equal(a_out, a_ref), rep
        assert torch.equal(g_out, g_ref), rep
        if r.n_out:
            assert torch.equal(r.state_out[: r.n_out], s_ref[: r.n_out]), rep
