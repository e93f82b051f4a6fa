"""Python binding of the C ABI (include/forkgdn.h): argument marshalling only.

Every function has the name of the C entry point it calls.  Tensors are
torch tensors on the current device; the stream is torch's current stream
unless one is given.  Nothing here computes any step of the method.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import _lib
from ._lib import FK_BF16, FK_F32, TreeMetaC, check

_DT = {torch.float32: FK_F32, torch.bfloat16: FK_BF16}


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    assert t.is_contiguous(), "tensors must be contiguous"
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


@dataclass
class TreeMeta:
    """A round's tree description: device int32 arrays plus host capacities
    (fields of ``fk_tree_meta``).  Build it with :func:`make_tree_meta`."""
    T: int
    S: int
    max_depth: int
    level_cap: int
    fork_cap: int
    n_pages: int
    n_state_in: int
    n_state_out: int
    tok_seg: torch.Tensor
    seg_parent: torch.Tensor
    seg_fork: torch.Tensor
    seg_cached_len: torch.Tensor
    seg_page_off: torch.Tensor
    seg_pages: torch.Tensor
    seg_state_in: torch.Tensor
    seg_state_out: torch.Tensor
    page_size: int = _lib.FK_TILE_TOKENS

    def c(self) -> TreeMetaC:
        m = TreeMetaC()
        for f in ("T", "S", "max_depth", "level_cap", "fork_cap", "page_size", "n_pages",
                  "n_state_in", "n_state_out"):
            setattr(m, f, int(getattr(self, f)))
        for f in ("tok_seg", "seg_parent", "seg_fork", "seg_cached_len", "seg_page_off",
                  "seg_pages", "seg_state_in", "seg_state_out"):
            t = getattr(self, f)
            setattr(m, f, t.data_ptr() if t is not None and t.numel() else
                    (t.data_ptr() if t is not None else None))
        return m


def make_tree_meta(tok_seg, seg_parent, seg_fork, seg_cached_len, seg_page_off, seg_pages,
                   n_pages, seg_state_in=None, seg_state_out=None, n_state_in=0, n_state_out=0,
                   max_depth=_lib.FK_MAX_DEPTH, level_cap=None, fork_cap=None,
                   device="cuda") -> TreeMeta:
    """Upload host int32 arrays of a round.  Capacities default to S (always
    sufficient); callers that know their rounds pass tighter ones."""
    S = len(seg_parent)

    def dev(a, n=None):
        a = np.ascontiguousarray(a if a is not None else np.full(n, -1), np.int32)
        if a.size == 0:
            a = np.zeros(1, np.int32)
        return torch.from_numpy(a).to(device)

    return TreeMeta(T=len(tok_seg), S=S, max_depth=max_depth, level_cap=level_cap or S,
                    fork_cap=fork_cap if fork_cap is not None else S, n_pages=n_pages,
                    n_state_in=n_state_in, n_state_out=n_state_out, tok_seg=dev(tok_seg),
                    seg_parent=dev(seg_parent), seg_fork=dev(seg_fork),
                    seg_cached_len=dev(seg_cached_len), seg_page_off=dev(seg_page_off),
                    seg_pages=dev(seg_pages), seg_state_in=dev(seg_state_in, S),
                    seg_state_out=dev(seg_state_out, S))


def fk_workspace_bytes(meta: TreeMeta, gdn_Hv: int = 0, gdn_dk: int = 0, gdn_dv: int = 0) -> int:
    m = meta.c()
    return int(_lib.load().fk_workspace_bytes(ctypes.byref(m), int(gdn_Hv), int(gdn_dk), int(gdn_dv)))


def alloc_workspace(meta: TreeMeta, gdn_Hv: int = 0, gdn_dk: int = 0, gdn_dv: int = 0,
                    device="cuda") -> torch.Tensor:
    """Workspace for a round and the largest GDN layer (Hv, dk, dv) it runs."""
    n = fk_workspace_bytes(meta, gdn_Hv, gdn_dk, gdn_dv)
    return torch.empty(n, dtype=torch.uint8, device=device)


def fk_tree_build(meta: TreeMeta, ws: torch.Tensor, stream=None):
    m = meta.c()
    check("fk_tree_build", _lib.load().fk_tree_build(ctypes.byref(m), _ptr(ws), ws.numel(),
                                                     _stream(stream)))


def fk_tree_validate_host(tok_seg, seg_parent, seg_fork, seg_cached_len, seg_page_off=None,
                          seg_pages=None, n_pages=0, seg_state_in=None, seg_state_out=None,
                          n_state_in=0, n_state_out=0, max_depth=_lib.FK_MAX_DEPTH,
                          level_cap=None, fork_cap=None) -> int:
    """Host-side validation of host int32 arrays; returns the status code."""
    S = len(seg_parent)
    keep = []

    def hp(a):
        if a is None:
            return None
        a = np.ascontiguousarray(a, np.int32)
        keep.append(a)
        return a.ctypes.data

    m = TreeMetaC()
    m.T, m.S, m.max_depth = len(tok_seg), S, max_depth
    m.level_cap = level_cap or max(S, 1)
    m.fork_cap = fork_cap if fork_cap is not None else S
    m.page_size, m.n_pages, m.n_state_in, m.n_state_out = _lib.FK_TILE_TOKENS, n_pages, n_state_in, n_state_out
    m.tok_seg, m.seg_parent, m.seg_fork = hp(tok_seg), hp(seg_parent), hp(seg_fork)
    m.seg_cached_len, m.seg_page_off, m.seg_pages = hp(seg_cached_len), hp(seg_page_off), hp(seg_pages)
    m.seg_state_in, m.seg_state_out = hp(seg_state_in), hp(seg_state_out)
    return int(_lib.load().fk_tree_validate_host(ctypes.byref(m)))


def fk_token_positions(meta: TreeMeta, ws: torch.Tensor, stream=None) -> torch.Tensor:
    pos = torch.empty(max(meta.T, 1), dtype=torch.int32, device=ws.device)
    m = meta.c()
    check("fk_token_positions", _lib.load().fk_token_positions(ctypes.byref(m), _ptr(ws), _ptr(pos),
                                                               _stream(stream)))
    return pos[:meta.T]


def kv_append(meta: TreeMeta, k, v, k_pool, v_pool, ws, stream=None):
    m = meta.c()
    check("kv_append", _lib.load().kv_append(ctypes.byref(m), _ptr(k), _ptr(v), _DT[k.dtype], k.shape[1],
                                             k.shape[2], _ptr(k_pool), _ptr(v_pool), _ptr(ws),
                                             _stream(stream)))


def fork_attn_forward(meta: TreeMeta, q, k, v, k_pool, v_pool, ws, scale=None, out=None,
                      stream=None) -> torch.Tensor:
    """k = v = None: the round's keys/values are already in the pool."""
    T, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    if out is None:
        out = torch.empty_like(q)
    scale = float(scale if scale is not None else d ** -0.5)
    m = meta.c()
    check("fork_attn_forward", _lib.load().fork_attn_forward(
        ctypes.byref(m), _ptr(q), _ptr(k), _ptr(v), _DT[q.dtype], Hq, Hkv, d, scale, _ptr(k_pool),
        _ptr(v_pool), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def fork_attn_forward_noalloc(meta: TreeMeta, q, k, v, k_pool, v_pool, scale=None, out=None, status=None,
                              stream=None) -> torch.Tensor:
    """fk_tree_build + fork_attn_forward without a workspace (the library's
    fixed per-GPU array holds the round's metadata); ``status`` (int32 device
    tensor of one element, optional) receives the round's status word."""
    T, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    if out is None:
        out = torch.empty_like(q)
    scale = float(scale if scale is not None else d ** -0.5)
    m = meta.c()
    check("fork_attn_forward_noalloc", _lib.load().fork_attn_forward_noalloc(
        ctypes.byref(m), _ptr(q), _ptr(k), _ptr(v), _DT[q.dtype], Hq, Hkv, d, scale, _ptr(k_pool), _ptr(v_pool),
        _ptr(out), _ptr(status), _stream(stream)))
    return out


def fork_attn_forward_rule(meta: TreeMeta, q, k, v, k_pool, v_pool, ws, rule, window=0, scale=None,
                           out=None, stream=None) -> torch.Tensor:
    """Attention under a visibility rule: _lib.FK_RULE_CAUSAL / FK_RULE_WINDOW
    (with ``window``) / FK_RULE_TWO_WAY.  k = v = None: K/V already paged."""
    T, Hq, d = q.shape
    Hkv = k_pool.shape[1]
    if out is None:
        out = torch.empty_like(q)
    scale = float(scale if scale is not None else d ** -0.5)
    m = meta.c()
    check("fork_attn_forward_rule", _lib.load().fork_attn_forward_rule(
        ctypes.byref(m), _ptr(q), _ptr(k), _ptr(v), _DT[q.dtype], Hq, Hkv, d, scale, int(rule), int(window),
        _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def fork_attn_readout(meta: TreeMeta, q_rows, rows, k_pool, v_pool, ws, rule=_lib.FK_RULE_CAUSAL, window=0,
                      scale=None, out=None, stream=None) -> torch.Tensor:
    """Attention at the stream tokens ``rows`` (int32 device tensor, -1 =
    unused) only; q_rows / out [n_rows, Hq, d].  K/V must already be paged."""
    n, Hq, d = q_rows.shape
    assert rows.dtype == torch.int32 and rows.numel() == n
    Hkv = k_pool.shape[1]
    if out is None:
        out = torch.zeros_like(q_rows)
    scale = float(scale if scale is not None else d ** -0.5)
    m = meta.c()
    check("fork_attn_readout", _lib.load().fork_attn_readout(
        ctypes.byref(m), _ptr(q_rows), _ptr(rows), n, _DT[q_rows.dtype], Hq, Hkv, d, scale, int(rule), int(window),
        _ptr(k_pool), _ptr(v_pool), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def gdn_fork_forward(meta: TreeMeta, q, k, v, a, b, ws, state_in=None, state_out=None, out=None,
                     stream=None) -> torch.Tensor:
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    if out is None:
        out = torch.empty_like(v)
    m = meta.c()
    check("gdn_fork_forward", _lib.load().gdn_fork_forward(
        ctypes.byref(m), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _DT[q.dtype], Hk, Hv, dk, dv,
        _ptr(state_in), _ptr(state_out), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def gdn_conv_forward(meta: TreeMeta, x, w, ws, window_in=None, window_out=None, out=None,
                     stream=None) -> torch.Tensor:
    """x [T, C], w [C, W] float; windows [slots, W-1, C] in x's dtype."""
    T, C = x.shape
    W = w.shape[1]
    if out is None:
        out = torch.empty_like(x)
    m = meta.c()
    check("gdn_conv_forward", _lib.load().gdn_conv_forward(
        ctypes.byref(m), _ptr(x), _DT[x.dtype], C, W, _ptr(w), _ptr(window_in), _ptr(window_out),
        _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
    return out


def gdn_checkpoint_save(state_out, slot, ckpt, count=1, stream=None):
    """Copy state_out[slot:slot+count] into ckpt ([count, Hv, dv, dk] or [Hv, dv, dk])."""
    n, Hv, dv, dk = state_out.shape
    assert ckpt.numel() == count * Hv * dv * dk
    check("gdn_checkpoint_save", _lib.load().gdn_checkpoint_save(
        _ptr(state_out), int(slot), int(count), n, Hv, dk, dv, _ptr(ckpt), _stream(stream)))


def gdn_checkpoint_resume(ckpt, state_in, slot, count=1, stream=None):
    """Copy saved states ckpt into state_in[slot:slot+count]."""
    n, Hv, dv, dk = state_in.shape
    assert ckpt.numel() == count * Hv * dv * dk
    check("gdn_checkpoint_resume", _lib.load().gdn_checkpoint_resume(
        _ptr(ckpt), _ptr(state_in), int(slot), int(count), n, Hv, dk, dv, _stream(stream)))


def fk_proj_gemm(x, w, rows=None, out=None, stream=None) -> torch.Tensor:
    """y[m] = x[rows[m]] @ w.T (rows None: every row of x); x [Mx, K], w [N, K]
    bf16; rows int32 device tensor [M] (-1 = unused entry, row untouched)."""
    Mx, K = x.shape
    N = w.shape[0]
    assert w.shape[1] == K
    M = Mx if rows is None else rows.numel()
    if rows is not None:
        assert rows.dtype == torch.int32
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    check("fk_proj_gemm", _lib.load().fk_proj_gemm(_ptr(x), Mx, _ptr(rows), M, K, _ptr(w), N, _DT[x.dtype],
                                                   _ptr(out), _stream(stream)))
    return out


def fk_read_status(ws, stream=None) -> int:
    v = ctypes.c_int32(0)
    check("fk_read_status", _lib.load().fk_read_status(_ptr(ws), _stream(stream), ctypes.byref(v)))
    return int(v.value)


def fk_strerror(code: int) -> str:
    return _lib.load().fk_strerror(int(code)).decode()


def fk_peak_mfma_bf16(n_wg: int, iters: int, sink=None, stream=None) -> float:
    """Launch the dense bf16 MFMA loop (a measurement utility) on `stream`;
    returns the launch's product flops.  The caller times it."""
    if sink is None:
        sink = torch.empty(n_wg, dtype=torch.float32, device="cuda")
    flops = ctypes.c_double(0.0)
    _lib.check("fk_peak_mfma_bf16", _lib.load().fk_peak_mfma_bf16(_ptr(sink), int(n_wg), int(iters),
                                                                  ctypes.byref(flops), _stream(stream)))
    return flops.value

