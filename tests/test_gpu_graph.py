"""A round recorded once as a HIP graph and replayed (Flide section 3.3.2:
pre-recorded execution graphs, every round-dependent value in device
buffers, one graph per capacity bucket, padding only at the tail).  Each
replay -- with other eager work and synchronisations in between -- must give
the eager run's bits; after the inputs are refilled in place, a replay must
give the bits of an eager run on the new values; and rounds with different
trees replayed through one bucket's graph each give the bits of their own
exact-size eager run."""
import numpy as np
import pytest
import torch

import gated_deltanet_amd as fk
from tests.harness import GpuRound, dev_tensor, state_slots
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


# --------------------------------------------------------------------------
# capacity buckets (Flide section 3.3.2: one graph per stream capacity,
# padding only at the tail)
# --------------------------------------------------------------------------

class BucketStep:
    """Device buffers of one capacity bucket (tree description, inputs,
    outputs, pools, states, workspace) and the step the graph records."""

    def __init__(self, bucket, page_cap=4096, n_pages=4096, n_slots=256):
        self.b = bucket
        self.tree = fk.BucketRound(bucket, page_cap, n_pages, n_state_in=n_slots, n_state_out=n_slots)
        self.ws = fk.alloc_workspace(self.tree.meta, SH.Hv, SH.dk, SH.dv)
        T = bucket.T
        self.x = {n: torch.zeros((T,) + SH.dims(n), dtype=torch.float32 if n in ("ga", "gb") else torch.bfloat16,
                                 device="cuda") for n in ("aq", "ak", "av", "gq", "gk", "gv", "ga", "gb")}
        self.k_pool = torch.zeros((n_pages, SH.Hkv, 16, SH.d), dtype=torch.bfloat16, device="cuda")
        self.v_pool = torch.zeros((n_pages, SH.Hkv, SH.d, 16), dtype=torch.bfloat16, device="cuda")
        self.a_out = torch.zeros_like(self.x["aq"])
        self.g_out = torch.zeros_like(self.x["gv"])
        self.state_in = torch.zeros((n_slots, SH.Hv, SH.dv, SH.dk), dtype=torch.float32, device="cuda")
        self.state_out = torch.zeros_like(self.state_in)

    def load(self, inp, state_in):
        """Refill every buffer in place with a round (its history K/V appended
        eagerly into pages 0.. first, as a resume does)."""
        t = inp.tree
        ts, par, fkk, cl = t.arrays()
        ssi, sso, n_in, _ = state_slots(t)
        cached = [i for i, s in enumerate(t.segs) if s.cached]
        hist_pages, nxt = {}, 0
        for s in cached:
            n = -(-t.segs[s].length // 16)
            hist_pages[s] = list(range(nxt, nxt + n))
            nxt += n
        if cached:
            hts = np.concatenate([np.full(t.segs[s].length, j, np.int32) for j, s in enumerate(cached)])
            hplan = fk.plan_round(hts, np.full(len(cached), -1), np.zeros(len(cached)), np.zeros(len(cached)),
                                  first_page=0, n_pages=self.tree.meta.n_pages)
            hws = fk.alloc_workspace(hplan.meta)
            fk.fk_tree_build(hplan.meta, hws)
            fk.kv_append(hplan.meta, dev_tensor(inp, "ak", True), dev_tensor(inp, "av", True), self.k_pool,
                         self.v_pool, hws)
            assert fk.fk_read_status(hws) == 0
        arrays, _, _, _ = fk.plan_arrays(ts, par, fkk, cl, cached_pages=hist_pages, first_page=nxt,
                                         seg_state_in=ssi, seg_state_out=sso, bucket=self.b)
        self.tree.load(arrays)
        for n, x in self.x.items():
            x.zero_()
            x[:t.T] = dev_tensor(inp, n)
        if n_in:
            self.state_in[:n_in] = torch.from_numpy(np.ascontiguousarray(state_in, np.float32)).cuda()
        self.a_out.fill_(float("nan"))
        self.g_out.fill_(float("nan"))
        self.state_out.fill_(float("nan"))
        torch.cuda.synchronize()

    def step(self):
        m, x = self.tree.meta, self.x
        fk.fk_tree_build(m, self.ws)
        fk.kv_append(m, x["ak"], x["av"], self.k_pool, self.v_pool, self.ws)
        fk.fork_attn_forward(m, x["aq"], None, None, self.k_pool, self.v_pool, self.ws, out=self.a_out)
        fk.gdn_fork_forward(m, x["gq"], x["gk"], x["gv"], x["ga"], x["gb"], self.ws, state_in=self.state_in,
                            state_out=self.state_out, out=self.g_out)


def _exact(r):
    """Eager outputs of the round described at its exact size."""
    a = r.attention().clone()
    g = r.gdn().clone()
    torch.cuda.synchronize()
    assert r.status() == 0
    return a, g, r.state_out[: r.n_out].clone()


def test_bucket_graph_replays_different_rounds():
    """Two rounds with different trees (stream length, segment count, depth,
    cached histories) refill one bucket's buffers and replay the one graph
    captured for it; each replay gives, for every live token and every final
    state, the bits of that round run eagerly at its exact size -- and a third
    replay of the first round gives them again."""
    rounds = []
    for seed, depth in ((41, 2), (42, 3)):
        rng = np.random.default_rng(seed)
        t = random_tree(rng, n_requests=3 + seed % 2, max_depth=depth, p_cached_root=0.5, p_internal_fork=0.4,
                        max_len=120)
        t.flatten()
        inp = draw_inputs(t, SH, seed, "bf16")
        n_in = sum(s.cached for s in t.segs)
        st = (rng.standard_normal((n_in, SH.Hv, SH.dv, SH.dk)) * 0.2).astype(np.float32) if n_in else None
        rounds.append((inp, st))
    trees = [inp.tree for inp, _ in rounds]
    assert len({(t.T, t.S) for t in trees}) == 2
    caps = [fk.capacities(*t.arrays()[1:]) for t in trees]
    bucket = fk.bucket_for(max(t.T for t in trees), max(t.S for t in trees), max(c[0] for c in caps),
                           max(c[1] for c in caps), max(c[2] for c in caps))
    print(f"[bucket graph] rounds T={[t.T for t in trees]} S={[t.S for t in trees]} bucket {bucket}", flush=True)
    fam = fk.GraphFamily(lambda b: BucketStep(b))
    for rep, k in enumerate((0, 1, 0)):
        inp, st = rounds[k]
        t = inp.tree
        a_ref, g_ref, s_ref = _exact(GpuRound(inp, state_in_np=st).build())
        obj, _ = fam.member(bucket)
        obj.load(inp, st)
        fam.replay(bucket)
        torch.cuda.synchronize()
        assert fk.fk_read_status(obj.ws) == 0
        assert torch.equal(obj.a_out[:t.T], a_ref), rep
        assert torch.equal(obj.g_out[:t.T], g_ref), rep
        assert torch.equal(obj.state_out[: len(s_ref)], s_ref), rep
        # padding rows are never written
        assert torch.isnan(obj.a_out[t.T:].float()).all() and torch.isnan(obj.g_out[t.T:].float()).all()
    assert len(fam.members) == 1


def test_padded_round_equals_exact_eager():
    """A round planned into a larger bucket (tail padding, unused segment
    slots) gives its exact-size bits on every entry point that reads the
    tree: the step, the short conv, the visibility rules, the selective
    readout (an entry naming a padding token is unused), and positions
    (-1 for padding)."""
    rng = np.random.default_rng(43)
    t = random_tree(rng, n_requests=4, max_depth=3, p_cached_root=0.4, p_internal_fork=0.4, max_len=100)
    t.flatten()
    inp = draw_inputs(t, SH, 43, "bf16")
    n_in = sum(s.cached for s in t.segs)
    st = (rng.standard_normal((n_in, SH.Hv, SH.dv, SH.dk)) * 0.2).astype(np.float32) if n_in else None
    r = GpuRound(inp, state_in_np=st).build()
    a_ref, g_ref, s_ref = _exact(r)
    caps = fk.capacities(*t.arrays()[1:])
    b = fk.Bucket(T=t.T + 300, S=t.S + 9, max_depth=8, level_cap=t.S + 9, fork_cap=caps[2] + 5)
    obj = BucketStep(b)
    obj.load(inp, st)
    obj.step()
    torch.cuda.synchronize()
    assert fk.fk_read_status(obj.ws) == 0
    assert torch.equal(obj.a_out[:t.T], a_ref)
    assert torch.equal(obj.g_out[:t.T], g_ref)
    assert torch.equal(obj.state_out[: len(s_ref)], s_ref)
    m = obj.tree.meta
    pos = fk.fk_token_positions(m, obj.ws)
    assert torch.equal(pos[:t.T], fk.fk_token_positions(r.meta, r.ws)) and bool((pos[t.T:] == -1).all())
    for rule, W in ((fk._lib.FK_RULE_WINDOW, 37), (fk._lib.FK_RULE_TWO_WAY, 0)):
        o = fk.fork_attn_forward_rule(m, obj.x["aq"], None, None, obj.k_pool, obj.v_pool, obj.ws, rule, W)
        assert torch.equal(o[:t.T], r.attention(rule=rule, window=W))
    C, W = 64, 4
    x = torch.randn((b.T, C), generator=torch.Generator(device="cuda").manual_seed(4), device="cuda")
    x = x.to(torch.bfloat16)
    x[t.T:] = 0
    w = torch.rand((C, W), generator=torch.Generator(device="cuda").manual_seed(5), device="cuda") - 0.5
    win_in = torch.zeros((256, W - 1, C), dtype=torch.bfloat16, device="cuda")
    y = fk.gdn_conv_forward(m, x, w, obj.ws, window_in=win_in,
                            window_out=torch.zeros((256, W - 1, C), dtype=torch.bfloat16, device="cuda"))
    y_ref = fk.gdn_conv_forward(r.meta, x[:t.T].contiguous(), w, r.ws, window_in=win_in[: max(n_in, 1)],
                                window_out=torch.zeros((max(r.n_out, 1), W - 1, C), dtype=torch.bfloat16,
                                                       device="cuda"))
    assert torch.equal(y[:t.T], y_ref)
    rows = torch.tensor([t.T - 1, t.T, b.T - 1, 0, -1], dtype=torch.int32, device="cuda")
    q_rows = obj.x["aq"][rows.clamp(min=0).long()].contiguous()
    out = torch.full_like(q_rows, 3.0)
    fk.fork_attn_readout(m, q_rows, rows, obj.k_pool, obj.v_pool, obj.ws, out=out)
    assert torch.equal(out[0], a_ref[t.T - 1]) and torch.equal(out[3], a_ref[0])
    assert bool((out[[1, 2, 4]] == 3.0).all())
