"""bf16 ForkAttention (MFMA kernel) against the fp64 oracle: max-abs 2e-2 and
mean-abs 2e-3 (bf16 inputs, fp32 accumulation, bf16 output), plus batch
invariance -- a branch's bits are the same alone and inside any round.  The
workloads at full size are in test_gpu_configs.py and test_gpu_resume.py."""
import numpy as np
import pytest
import torch

import gated_deltanet_amd as fk
from tests.harness import GpuRound, oracle_attention, to_f64
from workloads import random_tree, subtree_path
from workloads.tensors import Shapes, draw_inputs

pytestmark = pytest.mark.gpu
MAX_ABS, MEAN_ABS = 2e-2, 2e-3
SH = Shapes(16, 2, 128, 2, 4, 128, 128)


def _check(o, ref, sel=None):
    if sel is not None:
        o, ref = o[sel], ref[sel]
    err = np.abs(o - ref)
    assert np.isfinite(o).all()
    return err.max(), err.mean()


def _random(seed, **kw):
    rng = np.random.default_rng(1000 + seed)
    t = random_tree(rng, p_cached_root=0.4, p_internal_fork=0.4, max_len=90, **kw)
    if seed % 2:
        live = [i for i, s in enumerate(t.segs) if not s.cached]
        t.flatten(list(rng.permutation(live)))
    else:
        t.flatten()
    return draw_inputs(t, SH, 77 + seed, "bf16")


def test_attention_bf16_random_trees():
    for seed in range(10):
        inp = _random(seed)
        print(f"[attn bf16 random] seed {seed} T={inp.tree.T}", flush=True)
        r = GpuRound(inp).build()
        o = to_f64(r.attention())
        assert r.status() == 0
        mx, mean = _check(o, oracle_attention(inp))
        assert mx <= MAX_ABS and mean <= MEAN_ABS, (seed, mx, mean)


def test_attention_bf16_batch_invariance():
    """Every leaf's path asked alone (its chain, same boundaries) gives the
    bits it gets inside the round, under two different stream layouts."""
    rng = np.random.default_rng(5)
    t = random_tree(rng, n_requests=4, p_cached_root=0.3, p_internal_fork=0.3, max_len=70)
    t.flatten()
    inp = draw_inputs(t, SH, 4242, "bf16")
    full = to_f64(GpuRound(inp).build().attention())
    live = [i for i, s in enumerate(t.segs) if not s.cached]
    t2 = random_tree(np.random.default_rng(5), n_requests=4, p_cached_root=0.3, p_internal_fork=0.3,
                     max_len=70)
    t2.flatten(list(rng.permutation(live)))
    inp2 = draw_inputs(t2, SH, 4242, "bf16")
    perm = to_f64(GpuRound(inp2).build().attention())
    pos1 = {(int(s), i): x for x, (s, i) in enumerate(_local(t))}
    for x, key in enumerate(_local(t2)):
        assert np.array_equal(perm[x], full[pos1[key]])
    for leaf in t.leaves():
        sub, chain = subtree_path(t, leaf)
        sub.flatten()
        sub_inp = draw_inputs(sub, SH, 4242, "bf16", request_streams=[t.segs[leaf].request])
        alone = to_f64(GpuRound(sub_inp).build().attention())
        for x, (s, i) in enumerate(_local(sub)):
            assert np.array_equal(alone[x], full[pos1[(chain[s], i)]]), (leaf, s, i)


def _local(tree):
    out, starts = [], {}
    for t, s in enumerate(tree.tok_seg):
        starts.setdefault(int(s), t)
        out.append((int(s), t - starts[int(s)]))
    return out


def test_attention_bf16_run_twice_bitwise():
    inp = _random(3)
    r = GpuRound(inp).build()
    a1 = r.attention().clone()
    a2 = r.attention().clone()
    assert torch.equal(a1, a2)


def test_attention_bf16_kv_head_counts():
    """The K/V append moves 4, 2 or 1 kv heads of a page per block, whichever
    divides the kv head count: odd and even counts page and attend alike."""
    for seed, hkv in ((21, 1), (22, 3), (23, 6)):
        sh = Shapes(8 * hkv, hkv, 128, 2, 4, 128, 128)
        rng = np.random.default_rng(1000 + seed)
        t = random_tree(rng, n_requests=3, p_cached_root=0.4, p_internal_fork=0.4, max_len=60)
        t.flatten()
        inp = draw_inputs(t, sh, 77 + seed, "bf16")
        print(f"[attn bf16 kv heads] Hkv {hkv} T={t.T}", flush=True)
        r = GpuRound(inp).build()
        o = to_f64(r.attention())
        assert r.status() == 0
        mx, mean = _check(o, oracle_attention(inp))
        assert mx <= MAX_ABS and mean <= MEAN_ABS, (hkv, mx, mean)
