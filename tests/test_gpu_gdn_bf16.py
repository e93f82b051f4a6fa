"""bf16 chunked Gated DeltaNet (MFMA kernels, fp32 state) against the fp64
oracle -- max-abs 2e-2, mean-abs 2e-3 on outputs and final states -- plus
the invariants that only the GPU can show bitwise: batch invariance, the
fork-point state equals the trunk's own final state, and checkpoint resume
equals the full pass.  The workloads at full size are in test_gpu_configs.py
and test_gpu_resume.py."""
import numpy as np
import pytest
import torch

import gated_deltanet_amd as fk
from tests.harness import GpuRound, oracle_gdn, state_slots, to_f64
from workloads import build_tree, random_tree, subtree_path
from workloads.tensors import Shapes, draw_inputs

pytestmark = pytest.mark.gpu
MAX_ABS, MEAN_ABS = 2e-2, 2e-3
SH = Shapes(2, 1, 16, 2, 4, 128, 128)


def _err(o, ref):
    assert np.isfinite(o).all()
    d = np.abs(o - ref)
    return d.max(), d.mean()


def _random(seed, max_len=150, **kw):
    rng = np.random.default_rng(2000 + seed)
    t = random_tree(rng, p_cached_root=0.4, p_internal_fork=0.4, max_len=max_len, **kw)
    if seed % 2:
        live = [i for i, s in enumerate(t.segs) if not s.cached]
        t.flatten(list(rng.permutation(live)))
    else:
        t.flatten()
    inp = draw_inputs(t, SH, 91 + seed, "bf16")
    n_in = sum(s.cached for s in t.segs)
    st = (rng.standard_normal((n_in, SH.Hv, SH.dv, SH.dk)) * 0.2).astype(np.float32) if n_in else None
    return inp, st


def test_gdn_bf16_random_trees():
    for seed in range(10):
        inp, st_in = _random(seed)
        print(f"[gdn bf16 random] seed {seed} T={inp.tree.T} S={inp.tree.S}", flush=True)
        r = GpuRound(inp, state_in_np=st_in).build()
        o = to_f64(r.gdn())
        assert r.status() == 0
        ref, st_ref = oracle_gdn(inp, state_in=st_in)
        mx, mean = _err(o, ref)
        smx, smean = _err(to_f64(r.state_out)[: len(st_ref)], st_ref)
        print(f"  out {mx:.2e}/{mean:.2e} state {smx:.2e}/{smean:.2e}", flush=True)
        assert mx <= MAX_ABS and mean <= MEAN_ABS, (seed, mx, mean)
        assert smx <= MAX_ABS and smean <= MEAN_ABS, (seed, smx, smean)


def _local(tree):
    out, starts = [], {}
    for t, s in enumerate(tree.tok_seg):
        starts.setdefault(int(s), t)
        out.append((int(s), t - starts[int(s)]))
    return out


def test_gdn_bf16_batch_invariance():
    rng = np.random.default_rng(6)
    t = random_tree(rng, n_requests=4, p_cached_root=0.0, p_internal_fork=0.3, max_len=140)
    t.flatten()
    inp = draw_inputs(t, SH, 5151, "bf16")
    full = to_f64(GpuRound(inp).build().gdn())
    pos = {k: x for x, k in enumerate(_local(t))}
    live = [i for i, s in enumerate(t.segs) if not s.cached]
    t2 = random_tree(np.random.default_rng(6), n_requests=4, p_cached_root=0.0, p_internal_fork=0.3,
                     max_len=140)
    t2.flatten(list(rng.permutation(live)))
    perm = to_f64(GpuRound(draw_inputs(t2, SH, 5151, "bf16")).build().gdn())
    for x, key in enumerate(_local(t2)):
        assert np.array_equal(perm[x], full[pos[key]])
    for leaf in t.leaves():
        sub, chain = subtree_path(t, leaf)
        sub.flatten()
        alone = to_f64(GpuRound(draw_inputs(sub, SH, 5151, "bf16",
                                            request_streams=[t.segs[leaf].request])).build().gdn())
        for x, (s, i) in enumerate(_local(sub)):
            assert np.array_equal(alone[x], full[pos[(chain[s], i)]]), (leaf, s, i)


def test_gdn_bf16_fork_state_equals_trunk_final_state():
    """The state every child starts from is the trunk's own final state: a
    trunk-only round writes the same bits to state_out."""
    t = build_tree([[(-1, 0, 200), (0, None, 33), (0, None, 70), (0, 130, 20)]]).flatten()
    inp = draw_inputs(t, SH, 31, "bf16")
    r = GpuRound(inp).build()
    r.gdn()
    t1 = build_tree([[(-1, 0, 200)]]).flatten()
    r1 = GpuRound(draw_inputs(t1, SH, 31, "bf16")).build()
    r1.gdn()
    assert torch.equal(r.state_out[0], r1.state_out[0])
    # the internal fork at 130 sees exactly the state of a 130-token trunk
    t2 = build_tree([[(-1, 0, 130), (0, None, 20)]]).flatten()
    inp2 = draw_inputs(t2, SH, 31, "bf16")
    inp2.raw = {k: v.copy() for k, v in inp2.raw.items()}
    # same trunk values as the first 130 tokens of the 200-token trunk
    for k in inp.raw:
        inp2.raw[k][:130] = inp.raw[k][:130]
        inp2.raw[k][130:] = inp.raw[k][200 + 33 + 70:200 + 33 + 70 + 20]
    o_full = to_f64(r.gdn())
    o_chain = to_f64(GpuRound(inp2).build().gdn())
    # tokens of the internal-fork child: within tolerance (a 130-token trunk
    # is chunked 64+64+2, the fork point is a partial chunk of the 200 trunk)
    mx, mean = _err(o_chain[130:], o_full[200 + 33 + 70:])
    assert mx <= MAX_ABS and mean <= MEAN_ABS


def test_gdn_bf16_resume_equals_full_pass():
    """Checkpoint (Flide section 3.4): pass 1 runs the history live and saves
    its final state; pass 2 resumes from it as a cached segment.  The
    continuation's outputs and states are bitwise those of the full pass, and
    attention over the cached pages is bitwise too."""
    nodes_full = [(-1, 0, 300), (0, None, 100), (1, None, 40), (1, None, 25), (1, 60, 10)]
    tf = build_tree([nodes_full]).flatten()
    sh = Shapes(16, 2, 128, 2, 4, 128, 128)
    inp_f = draw_inputs(tf, sh, 808, "bf16")
    rf = GpuRound(inp_f).build()
    of, af = rf.gdn().clone(), rf.attention().clone()
    # pass 1: history alone
    th = build_tree([[(-1, 0, 300)]]).flatten()
    rh = GpuRound(draw_inputs(th, sh, 808, "bf16")).build()
    rh.gdn()
    ckpt = torch.empty_like(rh.state_out[0])
    fk.gdn_checkpoint_save(rh.state_out, 0, ckpt)
    # pass 2: resume
    tr = build_tree([[(-1, 0, 300, True)] + nodes_full[1:]]).flatten()
    inp_r = draw_inputs(tr, sh, 808, "bf16")
    rr = GpuRound(inp_r, state_in_np=np.zeros((1, sh.Hv, 128, 128), np.float32)).build()
    fk.gdn_checkpoint_resume(ckpt, rr.state_in, 0)
    orr, ar = rr.gdn(), rr.attention()
    tail = slice(300, tf.T)
    assert torch.equal(orr, of[tail])
    assert torch.equal(ar, af[tail])
    # states of the continuation's segments match the full pass bit for bit
    _, sso_f, _, _ = state_slots(tf)
    _, sso_r, _, _ = state_slots(tr)
    for s in range(1, tf.S):
        assert torch.equal(rr.state_out[sso_r[s]], rf.state_out[sso_f[s]])


def test_gdn_bf16_run_twice_bitwise():
    inp, st_in = _random(4)
    r = GpuRound(inp, state_in_np=st_in).build()
    a = r.gdn().clone()
    b = r.gdn().clone()
    assert torch.equal(a, b)
