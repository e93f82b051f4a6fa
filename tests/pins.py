"""Pins for the fp64 oracle: each check compares the oracle with something
other than itself -- brute force, a library routine, a closed form, or an
invariant the pages state.  Every check takes ``libpath`` so the mutation
test can run the same checks against oracle builds with a planted mistake.

Sources: Flide section 3.2 (Eq. 2 stream, per-token request/branch/position),
section 3.2.1 Eq. 3 (visibility), section 3.2.2 Eq. 4 (gated delta rule),
section 3.2.3 Proposition 3.1 (each branch equals its isolated pass),
section 3.4 (checkpoint resume computes the same function); the Flex page
section 2.1 Eq. 1 (softmax attention); ForkServe item 1 (deeper fan-out is
a sequence of aliases).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from workloads import build_tree, random_tree
from workloads.tensors import Shapes, draw_inputs

torch.set_num_threads(4)


# --------------------------------------------------------------------------
# brute-force helpers (independent of the oracle's path construction)
# --------------------------------------------------------------------------

def token_table(tree):
    """Per stream token: (segment, local index) by scanning the stream."""
    ts = tree.tok_seg
    seg_start = {}
    for t, s in enumerate(ts):
        seg_start.setdefault(int(s), t)
    return [(int(s), t - seg_start[int(s)]) for t, s in enumerate(ts)]


def brute_visible(tree):
    """Dense visibility over (history rows + stream tokens) by walking parents.

    Key y is visible to query x iff y's segment is x's segment or one of its
    ancestors; inside x's own segment y must not come later; inside a strict
    ancestor a, y must lie among the first ``fork`` tokens of a that the next
    segment on x's chain sees (the alias sequence of ForkServe item 1).
    Columns: history rows first (cached segments in index order), then stream.
    """
    segs = tree.segs
    tok = token_table(tree)
    hist_rows = []
    for i, s in enumerate(segs):
        if s.cached:
            hist_rows += [(i, j) for j in range(s.length)]
    keys = hist_rows + tok
    M = np.zeros((len(tok), len(keys)), bool)
    for x, (sx, ix) in enumerate(tok):
        limit = {sx: ix + 1}            # segment -> number of its tokens visible
        c = sx
        while segs[c].parent >= 0:
            limit[segs[c].parent] = segs[c].fork
            c = segs[c].parent
        for y, (sy, iy) in enumerate(keys):
            M[x, y] = sy in limit and iy < limit[sy]
    return M, len(hist_rows)


def eq3_visible(tree):
    """Flide Eq. 3 literally for depth-1 trees with forks at the trunk's end:
    j_y = j_x, c_y in {0, c_x}, t_y <= t_x, with (j, c, t) per token."""
    segs = tree.segs
    tok = token_table(tree)
    jct = []
    for (s, i) in tok:
        sg = segs[s]
        if sg.parent < 0:
            jct.append((sg.request, 0, i))
        else:
            jct.append((sg.request, s + 1, segs[sg.parent].length + i))
    T = len(tok)
    M = np.zeros((T, T), bool)
    for x in range(T):
        jx, cx, tx = jct[x]
        for y in range(T):
            jy, cy, ty = jct[y]
            M[x, y] = (jy == jx) and (cy in (0, cx)) and (ty <= tx)
    return M


def small_inputs(tree, seed=7, Hq=4, Hkv=2, d=16, Hk=2, Hv=4, dk=8, dv=8, dtype="f32"):
    return draw_inputs(tree, Shapes(Hq, Hkv, d, Hk, Hv, dk, dv), seed, dtype)


def run_attn(inp, mode=1, libpath=None, scale=None, tok_sel=None):
    ts, par, fk, cl = inp.tree.arrays()
    d = inp.shapes.d
    return oracle.attention(ts, par, fk, cl, inp.hist_off, inp.f64("aq"), inp.f64("ak"),
                            inp.f64("av"), inp.f64("ak", True), inp.f64("av", True),
                            scale if scale is not None else 1 / np.sqrt(d), mode=mode,
                            tok_sel=tok_sel, libpath=libpath)


def run_gdn(inp, mode=1, libpath=None, state_in=None, seg_state_in=None, seg_state_out=None,
            n_out=0, overrides=None):
    ts, par, fk, cl = inp.tree.arrays()
    arrs = {n: inp.f64(n) for n in ("gq", "gk", "gv", "ga", "gb")}
    if overrides:
        arrs.update(overrides)
    return oracle.gdn(ts, par, fk, cl, arrs["gq"], arrs["gk"], arrs["gv"], arrs["ga"], arrs["gb"],
                      state_in=state_in, seg_state_in=seg_state_in, seg_state_out=seg_state_out,
                      n_state_out=n_out, mode=mode, libpath=libpath)


def sdpa_masked(q, k, v, mask, scale):
    """torch fp64 CPU scaled_dot_product_attention with a boolean mask (GQA
    by repeating kv heads over contiguous groups).  q [T,Hq,d], k/v [N,Hkv,d]."""
    Hq, Hkv = q.shape[1], k.shape[1]
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)                       # [Hq,T,d]
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
    m = torch.from_numpy(mask)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return o.permute(1, 0, 2).numpy()


# --------------------------------------------------------------------------
# the pins
# --------------------------------------------------------------------------

def pin_closed_form_counts(libpath=None):
    """N_vis = sum over segments of len*pos0 + len(len+1)/2 per head; for the
    tiny request (trunk 48, branches 6/8/10) it is 1176+309+420+535 = 2440."""
    t = build_tree([[(-1, 0, 48), (0, None, 6), (0, None, 8), (0, None, 10)]]).flatten()
    ix = oracle.index(*t.arrays(), libpath=libpath)
    assert int((ix["tok_pos"].astype(np.int64) + 1).sum()) == 2440
    # agent fan-out session: trunk 4096 -> 4 x 256 -> each 4 x 32, ten sessions
    nodes = [(-1, 0, 4096)]
    for _ in range(4):
        nodes.append((0, None, 256))
        p = len(nodes) - 1
        nodes += [(p, None, 32)] * 4
    t = build_tree([nodes] * 10).flatten()
    ix = oracle.index(*t.arrays(), libpath=libpath)
    assert int((ix["tok_pos"].astype(np.int64) + 1).sum()) == 149_532_160
    t = build_tree([[(-1, 0, 32768)] + [(0, None, 64)] * 16] * 4).flatten()
    ix = oracle.index(*t.arrays(), libpath=libpath)
    assert int((ix["tok_pos"].astype(np.int64) + 1).sum()) == 2_281_900_032


def pin_positions_bruteforce(libpath=None, n=20):
    """Positions continue from the fork (Flide section 3.2): a token's position
    equals its number of visible keys minus one under the brute-force rule."""
    rng = np.random.default_rng(11)
    for _ in range(n):
        t = random_tree(rng, p_cached_root=0.3).flatten(order=None)
        M, nh = brute_visible(t)
        ix = oracle.index(*t.arrays(), libpath=libpath)
        np.testing.assert_array_equal(ix["tok_pos"] + 1, M.sum(1))


def visibility_probe(t, libpath=None, mode=1):
    """Read the oracle's visible sets through its attention: with q = 0 every
    visible key gets weight 1/|vis|, and one-hot values expose which keys."""
    M, nh = brute_visible(t)
    T, N = M.shape
    inp = small_inputs(t)
    q = np.zeros((T, 1, N))
    k = np.zeros((T, 1, N))
    v = np.eye(N)[nh:, None, :]
    hk = np.zeros((max(nh, 1), 1, N))
    hv = np.eye(N)[:nh, None, :] if nh else np.zeros((1, 1, N))
    ts, par, fk, cl = t.arrays()
    o, mism = oracle.attention(ts, par, fk, cl, inp.hist_off, q, k, v, hk, hv, 1.0, mode=mode,
                               libpath=libpath)
    return o[:, 0, :] > 0, M, mism


def pin_visibility_bruteforce(libpath=None, n=15):
    rng = np.random.default_rng(5)
    for i in range(n):
        t = random_tree(rng, p_cached_root=0.3, p_internal_fork=0.4)
        order = None
        if i % 2:   # any flat layout (Flide section 3.2.3)
            live = [j for j, s in enumerate(t.segs) if not s.cached]
            order = list(rng.permutation(live))
        t.flatten(order)
        for mode in (0, 1):
            vis, M, mism = visibility_probe(t, libpath, mode)
            np.testing.assert_array_equal(vis, M)
            assert mism == 0


def pin_visibility_eq3(libpath=None, n=10):
    """Depth-1 trees with end forks: the brute-force rule is Eq. 3 itself."""
    rng = np.random.default_rng(9)
    for _ in range(n):
        t = random_tree(rng, max_depth=1, p_internal_fork=0.0, max_fanout=4).flatten()
        vis, M, _ = visibility_probe(t, libpath)
        np.testing.assert_array_equal(vis, eq3_visible(t))


def pin_attention_single_path_sdpa(libpath=None):
    """A single path (a chain with end forks) equals plain causal attention:
    torch's fp64 scaled_dot_product_attention(is_causal=True)."""
    t = build_tree([[(-1, 0, 23), (0, None, 9), (1, None, 14)]]).flatten()
    inp = small_inputs(t, Hq=6, Hkv=2, d=12)
    o, _ = run_attn(inp, libpath=libpath)
    q, k, v = inp.f64("aq"), inp.f64("ak"), inp.f64("av")
    G = 3
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                           scale=1 / np.sqrt(12))
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def pin_attention_masked_sdpa(libpath=None, n=8):
    """Any tree: SDPA over the flat stream (history rows prepended) with the
    brute-force boolean mask."""
    rng = np.random.default_rng(3)
    for _ in range(n):
        t = random_tree(rng, p_cached_root=0.4, p_internal_fork=0.4).flatten()
        inp = small_inputs(t, Hq=4, Hkv=2, d=16, seed=int(rng.integers(1 << 30)))
        o, _ = run_attn(inp, libpath=libpath)
        M, nh = brute_visible(t)
        keys = np.concatenate([inp.f64("ak", True), inp.f64("ak")], 0)
        vals = np.concatenate([inp.f64("av", True), inp.f64("av")], 0)
        ref = sdpa_masked(inp.f64("aq"), keys, vals, M, 1 / 4.0)
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def pin_attention_closed_forms(libpath=None):
    """One visible key gives o = v; identical visible keys give the mean of
    their values."""
    t = build_tree([[(-1, 0, 10), (0, 4, 3)]]).flatten()
    inp = small_inputs(t, Hq=2, Hkv=1, d=8)
    q, k, v = inp.f64("aq"), inp.f64("ak").copy(), inp.f64("av")
    ts, par, fk, cl = t.arrays()
    o, _ = oracle.attention(ts, par, fk, cl, inp.hist_off, q, k, v, None, None, 0.35,
                            libpath=libpath)
    np.testing.assert_allclose(o[0, 0], v[0, 0], rtol=0, atol=1e-15)   # first trunk token
    k[:] = k[0]
    o, _ = oracle.attention(ts, par, fk, cl, inp.hist_off, q, k, v, None, None, 0.35,
                            libpath=libpath)
    # trunk token 5 sees trunk 0..5; branch token 1 sees trunk 0..3 and branch 0..1
    np.testing.assert_allclose(o[5, 1], v[0:6, 0].mean(0), rtol=0, atol=1e-14)
    br = [10, 11]
    exp_ = np.concatenate([v[0:4, 0], v[br, 0]], 0).mean(0)
    np.testing.assert_allclose(o[11, 0], exp_, rtol=0, atol=1e-14)


def pin_modes_agree(libpath=None, n=10):
    """Literal leaf-path runs and the per-segment/tree evaluation give the same
    bits; tokens shared by several leaf paths agree bit for bit."""
    rng = np.random.default_rng(21)
    for _ in range(n):
        t = random_tree(rng, p_cached_root=0.3, p_internal_fork=0.4).flatten()
        inp = small_inputs(t, seed=int(rng.integers(1 << 30)))
        o0, m0 = run_attn(inp, 0, libpath)
        o1, m1 = run_attn(inp, 1, libpath)
        assert m0 == 0 and np.array_equal(o0, o1)
        S = t.S
        cached = [i for i, s in enumerate(t.segs) if s.cached]
        ssi = np.full(S, -1)
        st = None
        if cached:
            ssi[cached] = np.arange(len(cached))
            st = rng.standard_normal((len(cached), inp.shapes.Hv, inp.shapes.dv, inp.shapes.dk)) * 0.3
        sso = np.arange(S)
        sso[cached] = -1
        g0 = run_gdn(inp, 0, libpath, st, ssi, sso, S)
        g1 = run_gdn(inp, 1, libpath, st, ssi, sso, S)
        assert g0[2] == 0
        assert np.array_equal(g0[0], g1[0])
        live = [i for i in range(S) if i not in cached]
        assert np.array_equal(g0[1][live], g1[1][live])


def _chain_tree(n_hist, lens):
    nodes = []
    if n_hist:
        nodes.append((-1, 0, n_hist, True))
    for i, L in enumerate(lens):
        p = len(nodes) - 1
        nodes.append((p, None, L))
    return build_tree([nodes]).flatten()


def pin_gdn_no_write(libpath=None):
    """b = 0 makes Eq. 4 a pure decay: S_t = (prod of a) S_0, o_t = S_t q_t."""
    t = _chain_tree(5, [7, 4])
    inp = small_inputs(t, Hk=2, Hv=4, dk=8, dv=6)
    rng = np.random.default_rng(1)
    S0 = rng.standard_normal((1, 4, 6, 8))
    b0 = np.zeros_like(inp.f64("gb"))
    o, _, _ = run_gdn(inp, 1, libpath, S0, np.array([0, -1, -1]), overrides={"gb": b0})
    a, q = inp.f64("ga"), inp.f64("gq")
    decay = np.cumprod(a, 0)                                           # [T, Hv]
    for h in range(4):
        ref = decay[:, h, None] * (q[:, h // 2, :] @ S0[0, h].T)
        np.testing.assert_allclose(o[:, h], ref, rtol=1e-13, atol=1e-14)
    t2 = _chain_tree(0, [6])
    inp2 = small_inputs(t2, Hk=2, Hv=4, dk=8, dv=6)
    o2, _, _ = run_gdn(inp2, 1, libpath, overrides={"gb": np.zeros_like(inp2.f64("gb"))})
    assert np.all(o2 == 0.0)


def pin_gdn_one_token(libpath=None):
    """From a zero state one token gives o = b (k . q) v."""
    t = _chain_tree(0, [1])
    inp = small_inputs(t, Hk=1, Hv=2, dk=8, dv=5)
    o, _, _ = run_gdn(inp, 1, libpath)
    q, k, v, b = inp.f64("gq")[0, 0], inp.f64("gk")[0, 0], inp.f64("gv")[0], inp.f64("gb")[0]
    ref = b[:, None] * (k @ q) * v
    np.testing.assert_allclose(o[0], ref, rtol=1e-14, atol=1e-15)


def pin_gdn_replace(libpath=None):
    """b = 1 with a unit key overwrites the memory at that key: S_t k_t = v_t
    for any a and earlier state (read back with q_t = k_t)."""
    t = _chain_tree(3, [12])
    inp = small_inputs(t, Hk=1, Hv=3, dk=8, dv=8)
    rng = np.random.default_rng(4)
    S0 = rng.standard_normal((1, 3, 8, 8))
    k = inp.f64("gk")
    k = k / np.sqrt((k * k).sum(-1, keepdims=True))     # exactly unit in fp64
    ov = {"gb": np.ones_like(inp.f64("gb")), "gq": k.copy(), "gk": k}
    o, _, _ = run_gdn(inp, 1, libpath, S0, np.array([0, -1]), overrides=ov)
    np.testing.assert_allclose(o, inp.f64("gv"), rtol=0, atol=1e-12)


def pin_gdn_orthonormal(libpath=None):
    """Orthonormal keys and b = 1 turn Eq. 4 into decayed linear attention:
    O = (Q K^T * D) V with D_tj = prod_{i=j+1..t} a_i (numpy matmul)."""
    L, dk, dv = 10, 16, 16
    t = _chain_tree(0, [4, 6])
    inp = small_inputs(t, Hk=1, Hv=2, dk=dk, dv=dv)
    rng = np.random.default_rng(8)
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    K = Qm[:L][:, None, :]
    ov = {"gk": K, "gb": np.ones_like(inp.f64("gb"))}
    o, _, _ = run_gdn(inp, 1, libpath, overrides=ov)
    q, v, a = inp.f64("gq")[:, 0], inp.f64("gv"), inp.f64("ga")
    for h in range(2):
        la = np.log(a[:, h])
        c = np.cumsum(la)
        D = np.tril(np.exp(c[:, None] - c[None, :]))
        ref = ((q @ K[:, 0].T) * D) @ v[:, h]
        np.testing.assert_allclose(o[:, h], ref, rtol=1e-11, atol=1e-12)


def brute_gdn(inp, state_in=None, seg_state_in=None):
    """Flat-stream brute force: every token's state comes from its predecessor
    on its own path (walk the stream by predecessor pointers), and the update
    is Eq. 4 in its matrix form S a (I - b k k^T) + b v k^T."""
    t = inp.tree
    segs = t.segs
    tok = token_table(t)
    start = {}
    for x, (s, i) in enumerate(tok):
        start.setdefault(s, x)
    Hk, Hv, dk, dv = inp.shapes.Hk, inp.shapes.Hv, inp.shapes.dk, inp.shapes.dv
    q, k, v, a, b = (inp.f64(n) for n in ("gq", "gk", "gv", "ga", "gb"))
    state = {}
    out = np.zeros((len(tok), Hv, dv))
    I = np.eye(dk)
    for x in range(len(tok)):
        pass
    done = set()

    def pred_state(x):
        s, i = tok[x]
        if i > 0:
            return state[start[s] + i - 1]
        p = segs[s].parent
        if p < 0:
            return np.zeros((Hv, dv, dk))
        if segs[p].cached:
            return state_in[seg_state_in[p]]
        f = segs[s].fork
        if f == 0:
            return pred_state_of_start(p)
        return state[start[p] + f - 1]

    def pred_state_of_start(s):
        return pred_state(start[s])

    order = sorted(range(len(tok)), key=lambda x: t.depth_of(tok[x][0]) * 10**6 + x)
    for x in order:
        S_prev = pred_state(x)
        S_new = np.zeros_like(S_prev)
        for h in range(Hv):
            g = h // (Hv // Hk)
            kk = k[x, g]
            S_new[h] = a[x, h] * S_prev[h] @ (I - b[x, h] * np.outer(kk, kk)) + b[x, h] * np.outer(v[x, h], kk)
            out[x, h] = S_new[h] @ q[x, g]
        state[x] = S_new
    return out


def pin_gdn_bruteforce(libpath=None, n=8):
    rng = np.random.default_rng(17)
    for _ in range(n):
        t = random_tree(rng, p_cached_root=0.4, p_internal_fork=0.4, max_len=12).flatten()
        inp = small_inputs(t, Hk=2, Hv=4, dk=6, dv=5, seed=int(rng.integers(1 << 30)))
        cached = [i for i, s in enumerate(t.segs) if s.cached]
        ssi = np.full(t.S, -1)
        st = None
        if cached:
            ssi[cached] = np.arange(len(cached))
            st = rng.standard_normal((len(cached), 4, 5, 6)) * 0.5
        o, _, _ = run_gdn(inp, 1, libpath, st, ssi)
        ref = brute_gdn(inp, st, ssi)
        np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)


def _two_branch():
    return build_tree([[(-1, 0, 30), (0, None, 7), (0, 12, 9), (1, None, 5)],
                       [(-1, 0, 11), (0, None, 4)]])


def pin_trunk_independent(libpath=None):
    """Trunk outputs do not depend on the branches (removing them changes no bit)."""
    full = _two_branch().flatten()
    inp = small_inputs(full)
    trunk_only = build_tree([[(-1, 0, 30)], [(-1, 0, 11)]]).flatten()
    inp_t = small_inputs(trunk_only)
    o_full, _ = run_attn(inp, 1, libpath)
    o_tr, _ = run_attn(inp_t, 1, libpath)
    g_full = run_gdn(inp, 1, libpath, seg_state_out=np.array([0, -1, -1, -1, 1, -1]), n_out=2)
    g_tr = run_gdn(inp_t, 1, libpath, seg_state_out=np.array([0, 1]), n_out=2)
    tr_tok = [x for x, s in enumerate(full.tok_seg) if s in (0, 4)]
    assert np.array_equal(o_full[tr_tok], o_tr)
    assert np.array_equal(g_full[0][tr_tok], g_tr[0])
    # the fork-point state equals the trunk's final state from a trunk-only run
    assert np.array_equal(g_full[1], g_tr[1])


def pin_sibling_permutation(libpath=None):
    """Permuting siblings (and requests) in the stream changes no output bit."""
    tree = _two_branch()
    a = small_inputs(tree.flatten())
    oa, _ = run_attn(a, 1, libpath)
    ga = run_gdn(a, 1, libpath)[0]
    perm_order = [4, 5, 2, 0, 3, 1]
    tree_b = _two_branch().flatten(perm_order)
    b = small_inputs(tree_b)
    ob, _ = run_attn(b, 1, libpath)
    gb = run_gdn(b, 1, libpath)[0]
    # map tokens by (segment, local index)
    ta, tb = token_table(tree.flatten()), token_table(tree_b)
    ia = {st: x for x, st in enumerate(ta)}
    idx = [ia[st] for st in tb]
    assert np.array_equal(ob, oa[idx])
    assert np.array_equal(gb, ga[idx])


def pin_resume_equals_full(libpath=None):
    """Checkpoint resume (Flide section 3.4): a pass that resumes from the
    saved history (K/V rows + fp32-exact state) equals the full pass."""
    full = build_tree([[(-1, 0, 20), (0, None, 9), (1, None, 4), (1, 3, 6)]]).flatten()
    inp = small_inputs(full)
    o_full, _ = run_attn(inp, 1, libpath)
    g_full, st_full, _ = run_gdn(inp, 1, libpath, seg_state_out=np.array([0, -1, -1, -1]), n_out=1)
    res = build_tree([[(-1, 0, 20, True), (0, None, 9), (1, None, 4), (1, 3, 6)]]).flatten()
    inp_r = small_inputs(res)
    # cached history rows are the trunk's rows (same seed stream/key)
    o_r, _ = run_attn(inp_r, 1, libpath)
    g_r, _, _ = run_gdn(inp_r, 1, libpath, state_in=st_full, seg_state_in=np.array([0, -1, -1, -1]))
    tail = [x for x, s in enumerate(full.tok_seg) if s != 0]
    assert np.array_equal(o_full[tail], o_r)
    assert np.array_equal(g_full[tail], g_r)


def pin_chain_merge(libpath=None):
    """A chain A -> B -> C with end forks equals one segment A+B+C."""
    t3 = build_tree([[(-1, 0, 9), (0, None, 6), (1, None, 5)]]).flatten()
    inp3 = small_inputs(t3)
    t1 = build_tree([[(-1, 0, 20)]]).flatten()
    inp1 = small_inputs(t1)
    for name in inp1.raw:
        inp1.raw[name] = inp3.raw[name].copy()
    assert np.array_equal(run_attn(inp3, 1, libpath)[0], run_attn(inp1, 1, libpath)[0])
    assert np.array_equal(run_gdn(inp3, 1, libpath)[0], run_gdn(inp1, 1, libpath)[0])



# --------------------------------------------------------------------------
# visibility variants (Flide section 3.2.1: a sliding-window layer adds
# t_x - t_y < W; appendix H: models that read each block both ways fork
# their state under the same rule without t_y <= t_x)
# --------------------------------------------------------------------------

def brute_positions(tree):
    """pos0 of every segment by summing forks up the parent chain."""
    pos0 = []
    for i in range(tree.S):
        acc, j = 0, i
        while tree.segs[j].parent >= 0:
            acc += tree.segs[j].fork
            j = tree.segs[j].parent
        pos0.append(acc)
    return pos0


def brute_visible_rule(tree, rule, window=0):
    """Dense visibility (history rows first, then the stream) under a rule:
    causal / causal and t_x - t_y < window / two-way (every token of the own
    segment, each ancestor's first `fork` tokens)."""
    segs = tree.segs
    tok = token_table(tree)
    pos0 = brute_positions(tree)
    hist_rows = []
    for i, sg in enumerate(segs):
        if sg.cached:
            hist_rows += [(i, j) for j in range(sg.length)]
    keys = hist_rows + tok
    M = np.zeros((len(tok), len(keys)), bool)
    for x, (sx, ix) in enumerate(tok):
        limit = {sx: segs[sx].length if rule == oracle.RULE_TWO_WAY else ix + 1}
        c = sx
        while segs[c].parent >= 0:
            limit[segs[c].parent] = segs[c].fork
            c = segs[c].parent
        for y, (sy, iy) in enumerate(keys):
            vis = sy in limit and iy < limit[sy]
            if rule == oracle.RULE_WINDOW:
                vis = vis and (pos0[sx] + ix) - (pos0[sy] + iy) < window
            M[x, y] = vis
    return M


def _rule_run(inp, rule, window, libpath):
    ts, par, fk, cl = inp.tree.arrays()
    return oracle.attention(ts, par, fk, cl, inp.hist_off, inp.f64("aq"), inp.f64("ak"), inp.f64("av"),
                            inp.f64("ak", True), inp.f64("av", True), 1 / np.sqrt(inp.shapes.d), mode=1,
                            rule=rule, window=window, libpath=libpath)[0]


def pin_window_masked_sdpa(libpath=None, n=8):
    """Sliding window on random trees (cached roots, internal forks): SDPA
    with the brute-force mask (ancestry, t_y <= t_x and t_x - t_y < W)."""
    rng = np.random.default_rng(31)
    for i in range(n):
        t = random_tree(rng, p_cached_root=0.4, p_internal_fork=0.4).flatten()
        inp = small_inputs(t, Hq=4, Hkv=2, d=16, seed=int(rng.integers(1 << 30)))
        W = [1, 2, 5, 17, 40][i % 5]
        o = _rule_run(inp, oracle.RULE_WINDOW, W, libpath)
        M = brute_visible_rule(t, oracle.RULE_WINDOW, W)
        keys = np.concatenate([inp.f64("ak", True), inp.f64("ak")], 0)
        vals = np.concatenate([inp.f64("av", True), inp.f64("av")], 0)
        ref = sdpa_masked(inp.f64("aq"), keys, vals, M, 1 / 4.0)
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def pin_two_way_masked_sdpa(libpath=None, n=8):
    """Two-way rule on random trees: SDPA with the brute-force block mask."""
    rng = np.random.default_rng(37)
    for _ in range(n):
        t = random_tree(rng, p_cached_root=0.4, p_internal_fork=0.4).flatten()
        inp = small_inputs(t, Hq=4, Hkv=2, d=16, seed=int(rng.integers(1 << 30)))
        o = _rule_run(inp, oracle.RULE_TWO_WAY, 0, libpath)
        M = brute_visible_rule(t, oracle.RULE_TWO_WAY)
        keys = np.concatenate([inp.f64("ak", True), inp.f64("ak")], 0)
        vals = np.concatenate([inp.f64("av", True), inp.f64("av")], 0)
        ref = sdpa_masked(inp.f64("aq"), keys, vals, M, 1 / 4.0)
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def pin_rule_special_cases(libpath=None):
    """One segment read both ways is plain non-causal SDPA (no mask); a
    window of 1 gives o = v of the token itself; a window longer than every
    path is the causal rule, bit for bit."""
    t = build_tree([[(-1, 0, 19)]]).flatten()
    inp = small_inputs(t, Hq=4, Hkv=2, d=12)
    o = _rule_run(inp, oracle.RULE_TWO_WAY, 0, libpath)
    q, k, v = inp.f64("aq"), inp.f64("ak"), inp.f64("av")
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(2, 0).contiguous()
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(2, 0).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=1 / np.sqrt(12))
    np.testing.assert_allclose(o, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)
    t = _two_branch().flatten()
    inp = small_inputs(t)
    o1 = _rule_run(inp, oracle.RULE_WINDOW, 1, libpath)
    v = inp.f64("av")
    for h in range(inp.shapes.Hq):
        np.testing.assert_allclose(o1[:, h], v[:, h // 2], rtol=0, atol=1e-15)
    big = _rule_run(inp, oracle.RULE_WINDOW, 10_000, libpath)
    assert np.array_equal(big, _rule_run(inp, oracle.RULE_CAUSAL, 0, libpath))


# --------------------------------------------------------------------------
# short causal convolution in front of the GDN rule (Flide section 3.2.2:
# the conv reads each token's predecessors through the tree index, so a
# question's first tokens see the last tokens of its state; section 3.4:
# a checkpoint keeps the conv window)
# --------------------------------------------------------------------------

def run_conv(tree, cin, libpath=None, seg_state_out=None, n_out=0, w=None):
    ts, par, fk, cl = tree.arrays()
    return oracle.conv(ts, par, fk, cl, cin.hist_off, cin.f64(), cin.f64(True),
                       cin.w if w is None else w, seg_state_out=seg_state_out,
                       n_state_out=n_out, libpath=libpath)


def brute_predecessors(tree, depth):
    """Per stream token, its 0..depth-th predecessors as ('s', token) /
    ('h', history row) / None, by walking the tree one step at a time: the
    previous token of the same segment, else the parent's token at index
    fork - 1, else (fork 0) the predecessor of the parent's first token."""
    segs = tree.segs
    tok = token_table(tree)
    start = {}
    for x, (sg, i) in enumerate(tok):
        start.setdefault(sg, x)
    hist_off = {}
    acc = 0
    for i, sg in enumerate(segs):
        if sg.cached:
            hist_off[i] = acc
            acc += sg.length

    def row(sg, i):
        return ("h", hist_off[sg] + i) if segs[sg].cached else ("s", start[sg] + i)

    def prev(sg, i):
        while True:
            if i > 0:
                return sg, i - 1
            p = segs[sg].parent
            if p < 0:
                return None
            sg, i = p, segs[sg].fork

    out = []
    for (sg, i) in tok:
        chain, cur = [row(sg, i)], (sg, i)
        for _ in range(depth):
            cur = prev(*cur) if cur is not None else None
            chain.append(row(*cur) if cur is not None else None)
        out.append(chain)
    return out


def _conv_tree_inputs(rng, C=5, W=4, **kw):
    t = random_tree(rng, **kw).flatten()
    from workloads import draw_conv
    return t, draw_conv(t, C, W, int(rng.integers(1 << 30)), "f32")


def pin_conv_bruteforce(libpath=None, n=12):
    """Random trees (cached roots, internal forks, fork 0): y_t = sum_i
    w[:, i] x_{pred_i(t)} with predecessors found by walking the tree."""
    rng = np.random.default_rng(23)
    for _ in range(n):
        W = int(rng.integers(1, 6))
        t, cin = _conv_tree_inputs(rng, C=4, W=W, p_cached_root=0.4, p_internal_fork=0.4, max_len=9)
        x, hx = cin.f64(), cin.f64(True)
        y, _ = run_conv(t, cin, libpath)
        ref = np.zeros_like(x)
        for tt, chain in enumerate(brute_predecessors(t, W - 1)):
            for i, src in enumerate(chain):
                if src is not None:
                    ref[tt] += cin.w[:, i] * (x[src[1]] if src[0] == "s" else hx[src[1]])
        np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def pin_conv_single_path_conv1d(libpath=None):
    """A chain (with forks at segment ends) is one causal sequence: torch's
    fp64 depthwise conv1d with W-1 zeros of left padding (weights flipped,
    conv1d being a cross-correlation)."""
    from workloads import draw_conv
    for W in (1, 2, 4):
        t = _chain_tree(0, [7, 5, 1, 6])
        cin = draw_conv(t, 6, W, 5 + W, "f32")
        y, _ = run_conv(t, cin, libpath)
        x = torch.from_numpy(cin.f64().T.copy())[None]                      # [1, C, T]
        wt = torch.from_numpy(cin.w.astype(np.float64)[:, ::-1].copy())[:, None, :]
        ref = torch.nn.functional.conv1d(x, wt, padding=W - 1, groups=6)[0, :, : t.T].T.numpy()
        np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


def pin_conv_closed_forms(libpath=None):
    """w = e_0 is the identity; w = e_j shifts by j rows along each path
    (zero before the path's first row)."""
    t = build_tree([[(-1, 0, 6), (0, None, 3), (0, 2, 4), (2, 0, 2)]]).flatten()
    from workloads import draw_conv
    cin = draw_conv(t, 3, 4, 99, "f32")
    x = cin.f64()
    for j in range(4):
        w = np.zeros((3, 4))
        w[:, j] = 1.0
        y, _ = run_conv(t, cin, libpath, w=w)
        for tt, chain in enumerate(brute_predecessors(t, 3)):
            src = chain[j]
            np.testing.assert_array_equal(y[tt], x[src[1]] if src is not None else 0.0)


def pin_conv_window_and_resume(libpath=None):
    """The window saved at a segment end holds its path's last W-1 inputs;
    a pass over a cached history equals the full pass (Flide section 3.4);
    trunk rows do not depend on the branches."""
    from workloads import draw_conv
    W = 4
    full = build_tree([[(-1, 0, 2), (0, None, 1), (1, None, 4), (1, 0, 3)]]).flatten()
    cin = draw_conv(full, 5, W, 31, "f32")
    y_full, win = run_conv(full, cin, libpath, seg_state_out=np.array([0, 1, 2, 3]), n_out=4)
    x = cin.f64()
    # trunk has 2 rows: window = [0, x0, x1]; trunk+1 = [x0, x1, x2]
    np.testing.assert_array_equal(win[0], np.stack([np.zeros(5), x[0], x[1]]))
    np.testing.assert_array_equal(win[1], x[0:3])
    # the fork-0 child of segment 1 (3 rows) sees the trunk: [x1, xc0.., ]
    c3 = [tt for tt, s in enumerate(full.tok_seg) if s == 3]
    np.testing.assert_array_equal(win[3], np.stack([x[c3[0]], x[c3[1]], x[c3[2]]]))
    # resume: the trunk and segment 1 as cached history rows
    res = build_tree([[(-1, 0, 2, True), (0, None, 1, True), (1, None, 4)]]).flatten()
    cr = draw_conv(res, 5, W, 31, "f32")
    y_r, _ = run_conv(res, cr, libpath)
    tail = [tt for tt, s in enumerate(full.tok_seg) if s == 2]
    assert np.array_equal(y_full[tail], y_r)
    # trunk rows alone
    tr = build_tree([[(-1, 0, 2), (0, None, 1)]]).flatten()
    ct = draw_conv(tr, 5, W, 31, "f32")
    y_t, _ = run_conv(tr, ct, libpath)
    head = [tt for tt, s in enumerate(full.tok_seg) if s < 2]
    assert np.array_equal(y_full[head], y_t)


# --------------------------------------------------------------------------
# projection (Flide section 3.5: fixed-order products; section 3.3.3: the
# last layer's products only at the readout rows)
# --------------------------------------------------------------------------

def pin_proj_matmul(libpath=None):
    """The projection equals numpy's matrix product of the same fp64 values
    (a library routine), on ragged sizes."""
    rng = np.random.default_rng(11)
    for M, K, N in ((1, 1, 1), (37, 48, 20), (5, 129, 3)):
        x = rng.standard_normal((M, K))
        w = rng.standard_normal((N, K))
        y = oracle.proj(x, w, libpath=libpath)
        np.testing.assert_allclose(y, np.matmul(x, w.T), rtol=1e-12, atol=1e-12)


def pin_proj_rows(libpath=None):
    """An index buffer gathers rows of the plain product (duplicates allowed),
    and an unused entry (-1) leaves its output row untouched."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((9, 16))
    w = rng.standard_normal((7, 16))
    rows = np.array([4, -1, 0, 8, 4, -1, 2], np.int32)
    y0 = np.full((len(rows), 7), 123.0)
    y = oracle.proj(x, w, rows=rows, y=y0, libpath=libpath)
    full = np.matmul(x, w.T)
    for m, r in enumerate(rows):
        if r < 0:
            assert np.all(y[m] == 123.0)
        else:
            np.testing.assert_allclose(y[m], full[r], rtol=1e-12, atol=1e-12)


def pin_proj_closed_forms(libpath=None):
    """Identity weights return x exactly; a one-hot weight row e_j returns
    column j of x exactly."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((6, 10))
    assert np.array_equal(oracle.proj(x, np.eye(10), libpath=libpath), x)
    w = np.zeros((3, 10))
    w[0, 9], w[1, 0], w[2, 4] = 1.0, 1.0, 1.0
    assert np.array_equal(oracle.proj(x, w, libpath=libpath), x[:, [9, 0, 4]])


ALL_PINS = [v for k, v in list(globals().items()) if k.startswith("pin_")]
