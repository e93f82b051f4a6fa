"""Edge cases of the forked paths against the fp64 oracle, on the bf16 MFMA
kernels (attention max-abs 2e-2 / mean-abs 2e-3; GDN the same) and on the
float32 kernels (max-abs 1e-4): the deepest chain the metadata allows,
forks at tile (16) and chunk (64) boundaries and at offset 0, several
children forking at one offset, one-token segments, a cached history
continued by a one-token root, a wide fan-out, and a round with no live
tokens at all."""
import numpy as np
import pytest
import torch

import gated_deltanet_amd as fk
from tests.harness import GpuRound, oracle_attention, oracle_gdn, state_slots, to_f64
from workloads import build_tree
from workloads.tensors import Shapes, draw_inputs

pytestmark = pytest.mark.gpu
BF16_MAX, BF16_MEAN = 2e-2, 2e-3
F32_TOL = 1e-4
SH_BF16 = Shapes(16, 2, 128, 2, 4, 128, 128)
SH_F32 = Shapes(4, 2, 64, 2, 4, 32, 32)

# (name, per-request node lists (parent_local, fork, length[, cached]))
TREES = [
    ("chain_depth8", [[(-1, 0, 65), (0, None, 16), (1, None, 1), (2, None, 17), (3, None, 64),
                       (4, None, 15), (5, None, 63), (6, None, 130)]]),
    ("internal_forks", [[(-1, 0, 200), (0, 0, 5), (0, 1, 3), (0, 16, 17), (0, 63, 1), (0, 64, 33),
                         (0, 64, 2), (0, 65, 16), (0, 128, 64), (0, 199, 7), (0, 200, 9)]]),
    ("one_token", [[(-1, 0, 1), (0, None, 1), (0, None, 1), (0, None, 1), (1, None, 1), (2, None, 1)]]),
    ("cached_history", [[(-1, 0, 100, True), (0, None, 1), (1, None, 1), (1, None, 64)],
                        [(-1, 0, 37, True), (0, None, 129), (1, 64, 3), (1, None, 16)]]),
    ("wide_fanout", [[(-1, 0, 17)] + [(0, None, 3)] * 40]),
]


def _inputs(nodes, shapes, dtype, seed):
    t = build_tree(nodes).flatten()
    return draw_inputs(t, shapes, seed, dtype)


def _state_in(inp, seed):
    n_in = sum(s.cached for s in inp.tree.segs)
    if not n_in:
        return None
    rng = np.random.default_rng(seed)
    sh = inp.shapes
    return (rng.standard_normal((n_in, sh.Hv, sh.dv, sh.dk)) * 0.2).astype(np.float32)


def _err(o, ref):
    assert np.isfinite(o).all()
    d = np.abs(o - ref)
    return d.max(), d.mean()


@pytest.mark.parametrize("name,nodes", TREES, ids=[t[0] for t in TREES])
def test_edges_bf16(name, nodes):
    inp = _inputs(nodes, SH_BF16, "bf16", 4242)
    st = _state_in(inp, 7)
    print(f"[edges bf16] {name} T={inp.tree.T} S={inp.tree.S}", flush=True)
    r = GpuRound(inp, state_in_np=st).build()
    a = to_f64(r.attention())
    g = to_f64(r.gdn())
    assert r.status() == 0
    mx, mean = _err(a, oracle_attention(inp))
    print(f"  attention {mx:.2e}/{mean:.2e}", flush=True)
    assert mx <= BF16_MAX and mean <= BF16_MEAN
    ref, st_ref = oracle_gdn(inp, state_in=st)
    mx, mean = _err(g, ref)
    smx, smean = _err(to_f64(r.state_out)[: len(st_ref)], st_ref)
    print(f"  gdn {mx:.2e}/{mean:.2e} states {smx:.2e}/{smean:.2e}", flush=True)
    assert mx <= BF16_MAX and mean <= BF16_MEAN
    assert smx <= BF16_MAX and smean <= BF16_MEAN


@pytest.mark.parametrize("name,nodes", TREES, ids=[t[0] for t in TREES])
def test_edges_f32(name, nodes):
    inp = _inputs(nodes, SH_F32, "f32", 4343)
    st = _state_in(inp, 8)
    print(f"[edges f32] {name} T={inp.tree.T}", flush=True)
    r = GpuRound(inp, state_in_np=st).build()
    a = to_f64(r.attention())
    g = to_f64(r.gdn())
    assert r.status() == 0
    assert np.abs(a - oracle_attention(inp)).max() <= F32_TOL
    ref, st_ref = oracle_gdn(inp, state_in=st)
    assert np.abs(g - ref).max() <= F32_TOL
    assert np.abs(to_f64(r.state_out)[: len(st_ref)] - st_ref).max() <= F32_TOL


def test_empty_round():
    """Only cached histories, no live token: every call succeeds and writes nothing."""
    inp = _inputs([[(-1, 0, 40, True)], [(-1, 0, 3, True)]], SH_BF16, "bf16", 1)
    assert inp.tree.T == 0
    print("[edges] empty round", flush=True)
    r = GpuRound(inp, state_in_np=np.zeros((2, 4, 128, 128), np.float32)).build()
    assert r.status() == 0
    assert r.attention().numel() == 0
    assert r.gdn().numel() == 0
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_pool_of_nan_before_append(dtype):
    """A pool allocated without clearing (here: every slot NaN) gives the same
    outputs as a zeroed one: kv_append zero-fills the slots past each
    segment's last token -- history pages included -- so the masked slots the
    attention reads in a partial last page are finite."""
    sh, name = (SH_BF16, "bf16") if dtype == "bf16" else (SH_F32, "f32")
    nodes = dict(TREES)["cached_history"]
    inp = _inputs(nodes, sh, name, 99)
    print(f"[edges nan pool {dtype}] T={inp.tree.T}", flush=True)
    ref = GpuRound(inp).build().attention()
    r = GpuRound(inp, pool_fill=float("nan")).build()
    o = r.attention()
    assert r.status() == 0
    assert torch.isfinite(o.float()).all()
    assert torch.equal(o, ref)
