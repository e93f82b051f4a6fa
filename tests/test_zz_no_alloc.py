"""fork_attn_forward_noalloc (for callers that cannot allocate: it keeps the
round's metadata in the library's own fixed device array instead of a
caller workspace) against fk_tree_build + fork_attn_forward on the same
inputs: the same bits, on two calls in a row, the second with a smaller
round; a round whose metadata exceeds the array is refused on the host."""
import numpy as np
import pytest
import torch

import gated_deltanet_amd as fk
from gated_deltanet_amd import _lib
from tests.harness import GpuRound
from workloads import random_tree
from workloads.tensors import Shapes, draw_inputs

pytestmark = pytest.mark.gpu
SH = Shapes(16, 2, 128, 2, 4, 128, 128)


def _noalloc(r, k, v, out, status):
    """The call through the C ABI (the binding only marshals arguments)."""
    try:
        fk.fork_attn_forward_noalloc(r.meta, r.x["aq"], k, v, r.k_pool, r.v_pool, out=out, status=status)
    except _lib.FkError as e:
        return e.code
    return 0


def _round(seed, n_requests, max_len):
    rng = np.random.default_rng(seed)
    t = random_tree(rng, n_requests=n_requests, p_cached_root=0.3, p_internal_fork=0.4, max_len=max_len)
    t.flatten()
    return GpuRound(draw_inputs(t, SH, seed, "bf16"))


def test_noalloc_equals_workspace_entry_point():
    status = torch.full((1,), 77, dtype=torch.int32, device="cuda")
    for seed, n_req, max_len in ((71, 6, 150), (72, 2, 40)):   # the second round is smaller
        r = _round(seed, n_req, max_len)
        print(f"[noalloc] seed {seed} T={r.inp.tree.T} S={r.inp.tree.S}", flush=True)
        ref = r.build().attention().clone()
        assert r.status() == 0
        # clear this round's own pages (the cached histories' pages, written
        # before the round, stay): the call must append the keys/values itself
        t = r.inp.tree
        first = sum(-(-s.length // 16) for s in t.segs if s.cached)
        r.k_pool[first:].zero_()
        r.v_pool[first:].zero_()
        out = torch.full_like(ref, float("nan"))
        assert _noalloc(r, r.x["ak"], r.x["av"], out, status) == 0
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        assert torch.equal(out, ref)


def test_noalloc_refuses_oversized_round():
    r = _round(73, 1, 20)
    m = r.meta
    big = fk.TreeMeta(T=m.T, S=m.S, max_depth=m.max_depth, level_cap=1 << 24, fork_cap=m.fork_cap,
                      n_pages=m.n_pages, n_state_in=m.n_state_in, n_state_out=m.n_state_out, tok_seg=m.tok_seg,
                      seg_parent=m.seg_parent, seg_fork=m.seg_fork, seg_cached_len=m.seg_cached_len,
                      seg_page_off=m.seg_page_off, seg_pages=m.seg_pages, seg_state_in=m.seg_state_in,
                      seg_state_out=m.seg_state_out)
    r.meta = big
    out = torch.empty_like(r.x["aq"])
    assert _lib.STATUS[_noalloc(r, r.x["ak"], r.x["av"], out, None)] == "FK_E_WORKSPACE"
