"""The expanding-history resume workload (64 requests, each a 16,384-token
history checkpointed by a GPU pass, 1,024 new tokens, then mixed trees of
32-token branches) at full size, in the launch configuration the bench
times.  Two requests carry host-drawn values so the fp64 oracle can check
them: the history checkpoint, the round's attention on stratified rows (the
first and last row of every 16-token tile of every question, and of every
8th tile of the new root; every head), the GDN outputs of four v-heads over
every token, and the saved state of the new root -- the oracle runs each
history from the zero state, so the checkpoint/resume path is checked against
a full pass.  Every leaf of those requests, run alone, must give the
mixture's bits (batch invariance, Flide section 3.5)."""
import numpy as np
import pytest
import torch

import gated_deltanet_amd as fk
import oracle
from tests.harness import GpuRound, state_slots, stratified_rows, to_f64
from workloads import build_tree, subtree_path
from workloads.configs import WORKLOADS, config_requests
from workloads.tensors import draw_inputs

pytestmark = pytest.mark.gpu
MAX_ABS, MEAN_ABS = 2e-2, 2e-3
SAMPLED = (0, 37)
CFG = WORKLOADS[4]
SH = CFG.shapes
G_HEADS = 4   # v heads the GDN oracle runs (the first ones)


def _err(o, ref):
    assert np.isfinite(o).all()
    d = np.abs(o - ref)
    return d.max(), d.mean()


@pytest.fixture(scope="module")
def wl():
    from bench import ResumeWorkload

    print(f"[resume] building the workload, sampled requests {SAMPLED}", flush=True)
    w = ResumeWorkload(sampled=SAMPLED)
    w.checkpoint()
    print("[resume] checkpoint pass done", flush=True)
    w.step()
    torch.cuda.synchronize()
    assert fk.fk_read_status(w.ws) == 0
    print("[resume] round done", flush=True)
    return w


_CACHE = {}


def _request(wl, r):
    if r not in _CACHE:
        _CACHE[r] = _request_uncached(wl, r)
    return _CACHE[r]


def _request_uncached(wl, r):
    """Request r alone (host values), its history state from the oracle, and
    the mixture's stream rows of its live tokens, in its own stream order."""
    t = build_tree([config_requests(4)[r]]).flatten()
    inp = draw_inputs(t, SH, CFG.seed, "bf16", CFG.mu_a, request_streams=[r])
    base = min(i for i, s in enumerate(wl.tree.segs) if s.request == r)
    rows = np.concatenate([np.arange(wl.starts[base + j], wl.starts[base + j] + t.segs[j].length)
                           for j in t.order])
    hsel = (np.arange(SH.Hv) < G_HEADS).astype(np.uint8)
    H = t.segs[0].length
    z = np.zeros(1, np.int32)
    _, st_h, _ = oracle.gdn(np.zeros(H, np.int32), z - 1, z, z, inp.f64("gq", True), inp.f64("gk", True),
                            inp.f64("gv", True), inp.f64("ga", True), inp.f64("gb", True),
                            seg_state_out=np.zeros(1, np.int32), n_state_out=1, mode=1, head_sel=hsel)
    return t, inp, rows, hsel, st_h, base


@pytest.mark.parametrize("r", SAMPLED)
def test_resume_matches_oracle(wl, r):
    t, inp, rows, hsel, st_h, base = _request(wl, r)
    slot = wl.hist.index(base)
    g = slice(0, G_HEADS)
    print(f"[resume r={r}] T={t.T} segments={t.S}", flush=True)
    # the checkpoint of the GPU's history pass
    ck = to_f64(wl.ckpt[slot])[g]
    mx, mean = _err(ck, st_h[0][g])
    print(f"  checkpoint {mx:.2e}/{mean:.2e}", flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS
    # attention on stratified rows (every head), history + round keys: the
    # first and last row of every tile of every question and of every 8th
    # tile of the new root
    sel = stratified_rows(t, trunk_every=8).astype(np.uint8)
    ts, par, fk_, cl = t.arrays()
    ref, _ = oracle.attention(ts, par, fk_, cl, inp.hist_off, inp.f64("aq"), inp.f64("ak"), inp.f64("av"),
                              inp.f64("ak", True), inp.f64("av", True), SH.d ** -0.5, mode=1, tok_sel=sel)
    o = to_f64(wl.attn_out[torch.from_numpy(rows[sel.astype(bool)]).cuda()])
    mx, mean = _err(o, ref[sel.astype(bool)])
    print(f"  attention {mx:.2e}/{mean:.2e} on {int(sel.sum())} rows", flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS
    # GDN on a head subset, resumed from the oracle's own history state
    ssi, sso, _, n_out = state_slots(t)
    go, gst, _ = oracle.gdn(ts, par, fk_, cl, inp.f64("gq"), inp.f64("gk"), inp.f64("gv"), inp.f64("ga"),
                            inp.f64("gb"), state_in=st_h, seg_state_in=ssi, seg_state_out=sso,
                            n_state_out=n_out, mode=1, head_sel=hsel)
    o = to_f64(wl.gdn_out[torch.from_numpy(rows).cuda()])[:, g]
    mx, mean = _err(o, go[:, g])
    print(f"  gdn {mx:.2e}/{mean:.2e}", flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS
    # the state saved for the next pass: the new root's final state
    root = t.children(0)[0]
    so = to_f64(wl.ckpt_next[slot])[g]
    mx, mean = _err(so, gst[sso[root]][g])
    print(f"  saved state {mx:.2e}/{mean:.2e}", flush=True)
    assert mx <= MAX_ABS and mean <= MEAN_ABS


@pytest.mark.parametrize("r", SAMPLED)
def test_resume_batch_invariance(wl, r):
    """A history checkpointed alone, and a leaf path resumed alone from it,
    give the mixture's bits."""
    t, inp, rows, _, _, base = _request(wl, r)
    slot = wl.hist.index(base)
    # the history as a round of its own
    th = build_tree([[(-1, 0, t.segs[0].length)]]).flatten()
    rh = GpuRound(draw_inputs(th, SH, CFG.seed, "bf16", CFG.mu_a, request_streams=[r])).build()
    rh.gdn()
    assert rh.status() == 0
    assert torch.equal(rh.state_out[0], wl.ckpt[slot]), "history state differs from the mixture's"
    ck = wl.ckpt[slot:slot + 1].cpu().numpy()
    pos = {}
    acc = 0
    for j in t.order:
        for i in range(t.segs[j].length):
            pos[(j, i)] = rows[acc]
            acc += 1
    a_mix, g_mix = wl.attn_out, wl.gdn_out
    leaves = t.leaves()
    cache = {}
    print(f"[resume alone r={r}] {len(leaves)} leaves", flush=True)
    for n, leaf in enumerate(leaves):
        sub, chain = subtree_path(t, leaf)
        sub.flatten()
        if n % 10 == 0:
            print(f"  leaf {n + 1}/{len(leaves)}: {leaf} chain {chain}", flush=True)
        ra = GpuRound(draw_inputs(sub, SH, CFG.seed, "bf16", CFG.mu_a, request_streams=[r], cache=cache),
                      state_in_np=ck).build()
        a = ra.attention(scale=SH.d ** -0.5)
        o = ra.gdn()
        assert ra.status() == 0
        idx = [pos[(chain[s], i)] for s in sub.order for i in range(sub.segs[s].length)]
        idx = torch.tensor(idx, device="cuda")
        assert torch.equal(a, a_mix[idx]), ("attention", r, leaf)
        assert torch.equal(o, g_mix[idx]), ("gdn", r, leaf)


def test_resume_two_streams_bitwise(wl):
    """The bench's overlapped step -- the GDN call and the checkpoint save on a
    second stream beside the K/V append and the attention -- gives the serial
    step's bits for the whole round (outputs and the saved states), eagerly
    and replayed from a graph."""
    print("[resume] serial step vs the two-stream step", flush=True)
    wl.step()
    torch.cuda.synchronize()
    ref = (wl.attn_out.clone(), wl.gdn_out.clone(), wl.ckpt_next.clone())
    outs = (wl.attn_out, wl.gdn_out, wl.ckpt_next)
    for o in outs:
        o.zero_()
    wl.step_overlapped()
    torch.cuda.synchronize()
    assert fk.fk_read_status(wl.ws) == 0
    assert all(torch.equal(a, b) for a, b in zip(outs, ref))
    graph = fk.StepGraph(wl.step_overlapped)
    for rep in range(2):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(outs, ref)), rep
