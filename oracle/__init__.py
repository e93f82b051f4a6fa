"""fp64 CPU oracle for exact state forking -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package.  The HIP library never links or calls it, and
it imports nothing from the HIP library's package.

The arithmetic lives in plain C (``forkgdn_oracle.c``); this module only
builds it with gcc and marshals numpy arrays (Flide, section 3.2, Eq. 3 and
Eq. 4; Proposition 3.1 -- every branch equals its isolated pass).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "forkgdn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

ERRORS = {0: "ok", -1: "arg", -2: "seg_range", -3: "noncontig", -4: "parent", -5: "cycle",
          -6: "fork", -7: "empty", -8: "cached"}


def build(force: bool = True, extra_flags=()) -> str:
    """Compile the oracle with gcc (fp64, no fast-math)."""
    out = _LIB if not extra_flags else _LIB.replace(".so", "_" + "_".join(
        f.strip("-").replace("=", "") for f in extra_flags) + ".so")
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(_SRC):
        cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-Wall", *extra_flags, "-o", out, _SRC, "-lm"]
        subprocess.check_call(cmd)
    return out


_lib_cache = {}


def lib(path: Optional[str] = None) -> ctypes.CDLL:
    path = path or _LIB
    if path not in _lib_cache:
        if not os.path.exists(path):
            build(force=False)
        L = ctypes.CDLL(path)
        i32p = ctypes.POINTER(ctypes.c_int32)
        i64p = ctypes.POINTER(ctypes.c_int64)
        f64p = ctypes.POINTER(ctypes.c_double)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        L.or_index.argtypes = [ctypes.c_int, ctypes.c_int, i32p, i32p, i32p, i32p,
                               i32p, i32p, i32p, i32p, i32p, i32p]
        L.or_attention.argtypes = [ctypes.c_int, ctypes.c_int, i32p, i32p, i32p, i32p, i64p,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                   ctypes.c_int, ctypes.c_int, f64p, f64p, f64p, f64p, f64p, ctypes.c_int, u8p, u8p, f64p, i64p]
        L.or_gdn.argtypes = [ctypes.c_int, ctypes.c_int, i32p, i32p, i32p, i32p,
                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                             f64p, f64p, f64p, f64p, f64p, f64p, i32p, ctypes.c_int, u8p,
                             f64p, i32p, f64p, i64p]
        L.or_conv.argtypes = [ctypes.c_int, ctypes.c_int, i32p, i32p, i32p, i32p, i64p,
                              ctypes.c_int, ctypes.c_int, f64p, f64p, f64p, i32p, ctypes.c_int,
                              f64p, f64p]
        L.or_proj.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, f64p, i32p, f64p, f64p]
        _lib_cache[path] = L
    return _lib_cache[path]


def _p(a, ct):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ct))


def _i32(a):
    return np.ascontiguousarray(a, np.int32)


def _f64(a):
    return np.ascontiguousarray(a, np.float64)


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle rejected the tree: {ERRORS.get(code, code)}")
        self.code = code
        self.kind = ERRORS.get(code, str(code))


def index(tok_seg, seg_parent, seg_fork, seg_cached_len, libpath=None):
    """Canonical indexing: per segment (start, len, pos0, depth, root), per token position."""
    tok_seg, seg_parent, seg_fork, seg_cached_len = map(_i32, (tok_seg, seg_parent, seg_fork, seg_cached_len))
    T, S = len(tok_seg), len(seg_parent)
    outs = [np.zeros(S, np.int32) for _ in range(5)] + [np.zeros(max(T, 1), np.int32)]
    rc = lib(libpath).or_index(T, S, _p(tok_seg, ctypes.c_int32), _p(seg_parent, ctypes.c_int32),
                               _p(seg_fork, ctypes.c_int32), _p(seg_cached_len, ctypes.c_int32),
                               *[_p(o, ctypes.c_int32) for o in outs])
    if rc:
        raise OracleError(rc)
    start, length, pos0, depth, root, tok_pos = outs
    return dict(seg_start=start, seg_len=length, seg_pos0=pos0, seg_depth=depth, seg_root=root,
                tok_pos=tok_pos[:T])


RULE_CAUSAL, RULE_WINDOW, RULE_TWO_WAY = 0, 1, 2


def attention(tok_seg, seg_parent, seg_fork, seg_cached_len, hist_off, q, k, v, hk, hv,
              scale, mode=1, tok_sel=None, head_sel=None, libpath=None, rule=RULE_CAUSAL, window=0):
    """GQA softmax attention along every isolated path (fp64).

    ``rule``: RULE_CAUSAL (t_y <= t_x), RULE_WINDOW (also t_x - t_y <
    ``window``), RULE_TWO_WAY (the whole own segment and each ancestor's
    visible prefix; mode 1 only).

    q [T,Hq,d], k/v [T,Hkv,d] stream rows; hk/hv [Nh,Hkv,d] cached-history
    rows, ``hist_off[s]`` = first history row of cached segment s.  Returns
    (out [T,Hq,d], n_path_mismatch).  Unselected rows/heads are NaN.
    """
    tok_seg, seg_parent, seg_fork, seg_cached_len = map(_i32, (tok_seg, seg_parent, seg_fork, seg_cached_len))
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    hk = _f64(hk) if hk is not None and len(hk) else np.zeros((1, Hkv, d))
    hv = _f64(hv) if hv is not None and len(hv) else np.zeros((1, Hkv, d))
    hist_off = np.ascontiguousarray(hist_off, np.int64)
    out = np.full((max(T, 1), Hq, d), np.nan)
    mism = np.zeros(1, np.int64)
    ts = None if tok_sel is None else np.ascontiguousarray(tok_sel, np.uint8)
    hs = None if head_sel is None else np.ascontiguousarray(head_sel, np.uint8)
    rc = lib(libpath).or_attention(T, len(seg_parent), _p(tok_seg, ctypes.c_int32),
                                   _p(seg_parent, ctypes.c_int32), _p(seg_fork, ctypes.c_int32),
                                   _p(seg_cached_len, ctypes.c_int32), _p(hist_off, ctypes.c_int64),
                                   Hq, Hkv, d, float(scale), int(rule), int(window), _p(q, ctypes.c_double),
                                   _p(k, ctypes.c_double), _p(v, ctypes.c_double),
                                   _p(hk, ctypes.c_double), _p(hv, ctypes.c_double), int(mode),
                                   _p(ts, ctypes.c_uint8), _p(hs, ctypes.c_uint8),
                                   _p(out, ctypes.c_double), _p(mism, ctypes.c_int64))
    if rc:
        raise OracleError(rc)
    return out[:T], int(mism[0])


def gdn(tok_seg, seg_parent, seg_fork, seg_cached_len, q, k, v, a, b, state_in=None,
        seg_state_in=None, seg_state_out=None, n_state_out=0, mode=1, head_sel=None,
        libpath=None):
    """Gated delta rule (Eq. 4) along every isolated path (fp64).

    q/k [T,Hk,dk], v [T,Hv,dv], a/b [T,Hv]; state_in [slots,Hv,dv,dk] for
    cached segments (``seg_state_in``).  Returns (out [T,Hv,dv],
    state_out [n_state_out,Hv,dv,dk], n_path_mismatch).
    """
    tok_seg, seg_parent, seg_fork, seg_cached_len = map(_i32, (tok_seg, seg_parent, seg_fork, seg_cached_len))
    q, k, v, a, b = map(_f64, (q, k, v, a, b))
    T, Hk, dk = q.shape
    Hv, dv = v.shape[1], v.shape[2]
    S = len(seg_parent)
    ssi = _i32(seg_state_in if seg_state_in is not None else np.full(S, -1))
    sso = _i32(seg_state_out if seg_state_out is not None else np.full(S, -1))
    st_in = _f64(state_in) if state_in is not None and len(state_in) else np.zeros((1, Hv, dv, dk))
    st_out = np.full((max(n_state_out, 1), Hv, dv, dk), np.nan)
    out = np.full((max(T, 1), Hv, dv), np.nan)
    mism = np.zeros(1, np.int64)
    hs = None if head_sel is None else np.ascontiguousarray(head_sel, np.uint8)
    rc = lib(libpath).or_gdn(T, S, _p(tok_seg, ctypes.c_int32), _p(seg_parent, ctypes.c_int32),
                             _p(seg_fork, ctypes.c_int32), _p(seg_cached_len, ctypes.c_int32),
                             Hk, Hv, dk, dv, *[_p(x, ctypes.c_double) for x in (q, k, v, a, b, st_in)],
                             _p(ssi, ctypes.c_int32), int(mode), _p(hs, ctypes.c_uint8),
                             _p(out, ctypes.c_double), _p(sso, ctypes.c_int32),
                             _p(st_out, ctypes.c_double), _p(mism, ctypes.c_int64))
    if rc:
        raise OracleError(rc)
    return out[:T], st_out[:n_state_out], int(mism[0])


def conv(tok_seg, seg_parent, seg_fork, seg_cached_len, hist_off, x, hx, w, seg_state_out=None,
         n_state_out=0, libpath=None):
    """Short causal convolution along every isolated path (fp64).

    x [T, C] stream rows, hx [Nh, C] cached-history rows (``hist_off`` as for
    attention), w [C, W] with w[:, i] applied to the i-th predecessor (i = 0:
    the token itself).  Returns (y [T, C], window_out [n_state_out, W-1, C]):
    the window of a segment with a ``seg_state_out`` slot is the input of the
    last W-1 rows of its isolated sequence, oldest first, zero where that
    sequence is shorter (Flide, section 3.2.2 and section 3.4).
    """
    tok_seg, seg_parent, seg_fork, seg_cached_len = map(_i32, (tok_seg, seg_parent, seg_fork, seg_cached_len))
    x, w = _f64(x), _f64(w)
    T, C = x.shape
    W = w.shape[1]
    hx = _f64(hx) if hx is not None and len(hx) else np.zeros((1, C))
    hist_off = np.ascontiguousarray(hist_off, np.int64)
    S = len(seg_parent)
    sso = _i32(seg_state_out if seg_state_out is not None else np.full(S, -1))
    y = np.full((max(T, 1), C), np.nan)
    win = np.zeros((max(n_state_out, 1), max(W - 1, 1), C))
    rc = lib(libpath).or_conv(T, S, _p(tok_seg, ctypes.c_int32), _p(seg_parent, ctypes.c_int32),
                              _p(seg_fork, ctypes.c_int32), _p(seg_cached_len, ctypes.c_int32),
                              _p(hist_off, ctypes.c_int64), C, W, _p(w, ctypes.c_double),
                              _p(x, ctypes.c_double), _p(hx, ctypes.c_double), _p(sso, ctypes.c_int32),
                              int(n_state_out), _p(y, ctypes.c_double), _p(win, ctypes.c_double))
    if rc:
        raise OracleError(rc)
    return y[:T], win[:n_state_out, : W - 1]


def proj(x, w, rows=None, y=None, libpath=None):
    """Projection y[m, n] = sum_k x[r(m), k] w[n, k] (fp64), r(m) = rows[m] or m;
    an entry rows[m] < 0 leaves row m of ``y`` as it was (NaN when ``y`` is
    not given).  x [Mx, K], w [N, K]; returns y [M, N]."""
    x, w = _f64(x), _f64(w)
    Mx, K = x.shape
    N = w.shape[0]
    assert w.shape[1] == K
    r = None if rows is None else _i32(rows)
    M = Mx if r is None else len(r)
    out = np.full((max(M, 1), N), np.nan) if y is None else np.ascontiguousarray(np.array(y, np.float64))
    rc = lib(libpath).or_proj(M, Mx, K, N, _p(x, ctypes.c_double), _p(r, ctypes.c_int32), _p(w, ctypes.c_double),
                              _p(out, ctypes.c_double))
    if rc:
        raise OracleError(rc)
    return out[:M]
