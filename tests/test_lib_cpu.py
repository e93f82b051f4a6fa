"""C-ABI library on the CPU: it loads, exports every symbol the header
declares, validates rounds on the host exactly like the oracle classifies
them, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import gated_deltanet_amd as fk
from gated_deltanet_amd import _lib
from tests.malformed import CASES, arrays
from workloads import make_config, random_tree

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ORACLE_TO_FK = {"seg_range": "FK_E_SEG_RANGE", "noncontig": "FK_E_NONCONTIG", "parent": "FK_E_PARENT",
                "cycle": "FK_E_CYCLE", "fork": "FK_E_FORK", "empty": "FK_E_EMPTY", "cached": "FK_E_CACHED"}


def header_functions():
    txt = open(os.path.join(ROOT, "include", "forkgdn.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", txt)) - {"if", "sizeof"})


def test_exports_every_declared_symbol():
    L = _lib.load()
    names = header_functions()
    assert set(names) == set(_lib.SYMBOLS), names
    for n in names:
        assert hasattr(L, n), n
    assert L.fk_abi_version() == 1
    # the Python binding carries the same names (host-only helpers aside)
    for n in names:
        if n not in ("fk_abi_version",):
            assert callable(getattr(fk, n, None)), f"binding lacks {n}"


def test_strerror_covers_codes():
    for code, name in _lib.STATUS.items():
        assert fk.fk_strerror(code) not in ("", "unknown status"), name


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_host_validator_matches_oracle_classes(case):
    ts, par, fkk, cl, kind = arrays(case)
    ssi = np.where(cl > 0, 0, -1)    # cached segments bring a state: only the tree is wrong
    rc = fk.fk_tree_validate_host(ts, par, fkk, cl, max_depth=8, seg_state_in=ssi, n_state_in=1)
    assert _lib.STATUS[rc] == ORACLE_TO_FK[kind]


def test_host_validator_accepts_configs_and_random_trees():
    for i in range(4):
        _, t = make_config(i)
        ts, par, fkk, cl = t.arrays()
        assert fk.fk_tree_validate_host(ts, par, fkk, cl) == 0
    rng = np.random.default_rng(2)
    for _ in range(30):
        t = random_tree(rng, p_cached_root=0.3, p_internal_fork=0.4).flatten()
        ts, par, fkk, cl = t.arrays()
        ssi = np.where(cl > 0, 0, -1)
        assert fk.fk_tree_validate_host(ts, par, fkk, cl, seg_state_in=ssi, n_state_in=1) == 0


def test_host_validator_capacities_slots_pages():
    t = make_config(0)[1]
    ts, par, fkk, cl = t.arrays()
    assert _lib.STATUS[fk.fk_tree_validate_host(ts, par, fkk, cl, level_cap=2)] == "FK_E_CAPACITY"
    assert _lib.STATUS[fk.fk_tree_validate_host(ts, par, fkk, cl, fork_cap=0)] == "FK_E_CAPACITY"
    assert _lib.STATUS[fk.fk_tree_validate_host(ts, par, fkk, cl, max_depth=1)] == "FK_E_CYCLE"
    sso = np.array([0, -1, -1, 5])
    assert _lib.STATUS[fk.fk_tree_validate_host(ts, par, fkk, cl, seg_state_out=sso,
                                                n_state_out=2)] == "FK_E_STATE_SLOT"
    off = np.array([0, 3, 4, 5, 6])        # trunk of 48 needs 3 pages of 16
    pages = np.arange(6)
    assert fk.fk_tree_validate_host(ts, par, fkk, cl, off, pages, n_pages=6) == 0
    assert _lib.STATUS[fk.fk_tree_validate_host(ts, par, fkk, cl, off, pages, n_pages=5)] == "FK_E_PAGES"
    short = np.array([0, 2, 3, 4, 5])
    assert _lib.STATUS[fk.fk_tree_validate_host(ts, par, fkk, cl, short, pages, n_pages=6)] == "FK_E_PAGES"
    # a live child of a cached history needs a state slot
    ts2, par2, fk2, cl2 = np.array([1, 1], np.int32), np.array([-1, 0]), np.array([0, 4]), np.array([4, 0])
    assert _lib.STATUS[fk.fk_tree_validate_host(ts2, par2, fk2, cl2)] == "FK_E_STATE_SLOT"
    assert fk.fk_tree_validate_host(ts2, par2, fk2, cl2, seg_state_in=np.array([0, -1]), n_state_in=1) == 0


def test_workspace_bytes_grow_with_round():
    m = _lib.TreeMetaC()
    m.T, m.S, m.max_depth, m.level_cap, m.fork_cap, m.page_size = 100, 4, 2, 3, 1, 16
    L = _lib.load()
    a = L.fk_workspace_bytes(ctypes.byref(m), 0, 0, 0)
    b = L.fk_workspace_bytes(ctypes.byref(m), 2, 32, 32)
    # one fork-point state plus two 64 x 64 bf16 matrices per chunk and v-head
    assert b - a >= 2 * 32 * 32 * 4 + 2 * (2 + 4) * 2 * 64 * 64 * 2 and a > 0


def test_bad_arguments_rejected_on_host():
    L = _lib.load()
    assert L.fk_tree_build(None, None, 0, None) == -1
    assert L.gdn_checkpoint_save(ctypes.c_void_p(16), 3, 1, 2, 1, 16, 16, ctypes.c_void_p(16), None) == -1
    assert L.gdn_checkpoint_save(ctypes.c_void_p(16), 1, 2, 2, 1, 16, 16, ctypes.c_void_p(16), None) == -1
    assert L.gdn_checkpoint_resume(None, ctypes.c_void_p(16), 0, 1, 1, 1, 16, 16, None) == -1
    assert L.gdn_checkpoint_resume(ctypes.c_void_p(16), ctypes.c_void_p(16), 0, 0, 1, 1, 16, 16, None) == -1
    m = _lib.TreeMetaC()
    m.T, m.S, m.max_depth, m.level_cap, m.fork_cap, m.page_size = 0, 1, 1, 1, 0, 16
    assert L.gdn_fork_forward(ctypes.byref(m), None, None, None, None, None, 0, 1, 1, 48, 48, None,
                              None, None, ctypes.c_void_p(256), 1 << 20, None) == -1  # no seg arrays


def test_proj_gemm_host_errors():
    """Argument errors are reported on the host before anything is enqueued
    (no GPU call): unsupported widths, negative sizes, missing pointers; an
    empty batch is a no-op."""
    L = _lib.load()
    bf16, f32 = _lib.FK_BF16, _lib.FK_F32
    p = 16   # a dummy non-null address (never dereferenced on these paths)
    assert L.fk_proj_gemm(p, 4, None, 4, 64, p, 128, f32, p, None) == -2     # dtype
    assert L.fk_proj_gemm(p, 4, None, 4, 48, p, 128, bf16, p, None) == -2    # K % 64
    assert L.fk_proj_gemm(p, 4, None, 4, 64, p, 96, bf16, p, None) == -2     # N % 128
    assert L.fk_proj_gemm(p, 4, None, -1, 64, p, 128, bf16, p, None) == -1   # M < 0
    assert L.fk_proj_gemm(p, 4, None, 5, 64, p, 128, bf16, p, None) == -1    # M > Mx, no rows
    assert L.fk_proj_gemm(None, 4, None, 4, 64, p, 128, bf16, p, None) == -1
    assert L.fk_proj_gemm(None, 0, None, 0, 64, None, 128, bf16, None, None) == 0   # empty


def test_host_validator_padding_and_unused_slots():
    """A round planned into a larger capacity bucket (tail padding, unused
    segment slots) validates, with the same rules as the exact round; padding
    before a live token, tokens in an unused slot, and an unused slot as a
    parent are rejected."""
    rng = np.random.default_rng(8)
    for _ in range(20):
        t = random_tree(rng, p_cached_root=0.3, p_internal_fork=0.4).flatten()
        ts, par, fkk, cl = t.arrays()
        ssi = np.where(cl > 0, 0, -1)
        caps = fk.capacities(par, fkk, cl)
        b = fk.bucket_for(len(ts), len(par), *caps)
        a, _, _, _ = fk.plan_arrays(ts, par, fkk, cl, seg_state_in=ssi, bucket=b)
        assert len(a["tok_seg"]) == b.T >= len(ts) and len(a["seg_parent"]) == b.S >= len(par)
        assert fk.fk_tree_validate_host(a["tok_seg"], a["seg_parent"], a["seg_fork"], a["seg_cached_len"],
                                        seg_state_in=a["seg_state_in"], n_state_in=1, max_depth=b.max_depth,
                                        level_cap=b.level_cap, fork_cap=b.fork_cap) == 0
    ts = np.array([0, 0, -1, -1], np.int32)
    par, fkk = np.array([-1, -1]), np.array([0, 0])
    cl = np.array([0, -1])
    assert fk.fk_tree_validate_host(ts, par, fkk, cl) == 0
    bad = np.array([0, -1, 0, -1], np.int32)       # padding before a live token
    assert _lib.STATUS[fk.fk_tree_validate_host(bad, par, fkk, cl)] == "FK_E_SEG_RANGE"
    bad = np.array([0, 0, 1, -1], np.int32)        # a token in an unused slot
    assert _lib.STATUS[fk.fk_tree_validate_host(bad, par, fkk, cl)] == "FK_E_EMPTY"
    assert _lib.STATUS[fk.fk_tree_validate_host(ts, np.array([1, -1]), np.array([0, 0]), cl)] == "FK_E_PARENT"


def test_bucket_ladder():
    b = fk.bucket_for(24526, 117, 2, 101, 16)
    assert b.T >= 24526 and b.T < 1.25 * 24526 + 1024 and b.S >= 117 and b.max_depth == 2
    assert fk.bucket_for(1, 1, 1, 1, 0) == fk.Bucket(T=1024, S=16, max_depth=2, level_cap=16, fork_cap=16)
    # every member fits the round it was chosen for, and a larger round never gets a smaller member
    prev = None
    for T in (1000, 5000, 40000, 220640):
        b = fk.bucket_for(T, T // 40, 3, T // 50, T // 200)
        assert b.T >= T and b.S >= T // 40 and b.max_depth == 4
        if prev:
            assert b.T >= prev.T
        prev = b
