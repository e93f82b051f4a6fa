"""ctypes view of libforkgdn.so (include/forkgdn.h).  Loading fails loudly
when the library is missing: there is no fallback path."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libforkgdn.so")

FK_F32, FK_BF16 = 0, 1
FK_MAX_DEPTH = 8
FK_TILE_TOKENS = 16
FK_GDN_CHUNK = 64
FK_CONV_MAX_W = 8
FK_RULE_CAUSAL, FK_RULE_WINDOW, FK_RULE_TWO_WAY = 0, 1, 2

STATUS = {0: "FK_OK", -1: "FK_E_INVALID_ARG", -2: "FK_E_UNSUPPORTED", -3: "FK_E_WORKSPACE",
          -4: "FK_E_HIP", -10: "FK_E_SEG_RANGE", -11: "FK_E_NONCONTIG", -12: "FK_E_PARENT",
          -13: "FK_E_CYCLE", -14: "FK_E_FORK", -15: "FK_E_EMPTY", -16: "FK_E_CACHED",
          -17: "FK_E_PAGES", -18: "FK_E_CAPACITY", -19: "FK_E_STATE_SLOT"}

# exported symbols, in header order
SYMBOLS = ("fk_workspace_bytes", "fk_tree_build", "fk_tree_validate_host", "fk_token_positions",
           "kv_append", "fork_attn_forward", "fork_attn_forward_noalloc", "fork_attn_forward_rule", "fork_attn_readout", "gdn_fork_forward", "gdn_conv_forward", "gdn_checkpoint_save",
           "gdn_checkpoint_resume", "fk_proj_gemm", "fk_read_status", "fk_strerror", "fk_abi_version",
           "fk_peak_mfma_bf16")

_i32p = ctypes.POINTER(ctypes.c_int32)


class TreeMetaC(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("S", ctypes.c_int32), ("max_depth", ctypes.c_int32),
                ("level_cap", ctypes.c_int32), ("fork_cap", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("n_pages", ctypes.c_int32),
                ("n_state_in", ctypes.c_int32), ("n_state_out", ctypes.c_int32),
                ("tok_seg", ctypes.c_void_p), ("seg_parent", ctypes.c_void_p),
                ("seg_fork", ctypes.c_void_p), ("seg_cached_len", ctypes.c_void_p),
                ("seg_page_off", ctypes.c_void_p), ("seg_pages", ctypes.c_void_p),
                ("seg_state_in", ctypes.c_void_p), ("seg_state_out", ctypes.c_void_p)]


class FkError(RuntimeError):
    def __init__(self, fn, code):
        self.code = code
        self.name = STATUS.get(code, str(code))
        super().__init__(f"{fn} failed: {self.name}")


_LIB = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python gated_deltanet_amd/build.py` "
            "(the HIP library is the only implementation)")
    L = ctypes.CDLL(path)
    vp, sz, i32, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
    mp = ctypes.POINTER(TreeMetaC)
    L.fk_workspace_bytes.argtypes = [mp, i32, i32, i32]
    L.fk_workspace_bytes.restype = sz
    L.fk_tree_build.argtypes = [mp, vp, sz, vp]
    L.fk_tree_validate_host.argtypes = [mp]
    L.fk_token_positions.argtypes = [mp, vp, vp, vp]
    L.kv_append.argtypes = [mp, vp, vp, i32, i32, i32, vp, vp, vp, vp]
    L.fork_attn_forward.argtypes = [mp, vp, vp, vp, i32, i32, i32, i32, f32, vp, vp, vp, vp, sz, vp]
    L.fork_attn_forward_noalloc.argtypes = [mp, vp, vp, vp, i32, i32, i32, i32, f32, vp, vp, vp, vp, vp]
    L.fork_attn_forward_rule.argtypes = [mp, vp, vp, vp, i32, i32, i32, i32, f32, i32, i32, vp, vp, vp, vp, sz,
                                         vp]
    L.fork_attn_readout.argtypes = [mp, vp, vp, i32, i32, i32, i32, i32, f32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.gdn_fork_forward.argtypes = [mp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, vp, vp, sz, vp]
    L.gdn_conv_forward.argtypes = [mp, vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    L.gdn_checkpoint_save.argtypes = [vp, i32, i32, i32, i32, i32, i32, vp, vp]
    L.gdn_checkpoint_resume.argtypes = [vp, vp, i32, i32, i32, i32, i32, i32, vp]
    L.fk_proj_gemm.argtypes = [vp, i32, vp, i32, i32, vp, i32, i32, vp, vp]
    L.fk_read_status.argtypes = [vp, vp, _i32p]
    L.fk_peak_mfma_bf16.argtypes = [vp, i32, i32, ctypes.POINTER(ctypes.c_double), vp]
    L.fk_strerror.argtypes = [ctypes.c_int]
    L.fk_strerror.restype = ctypes.c_char_p
    for name in SYMBOLS:
        if name not in ("fk_workspace_bytes", "fk_strerror"):
            getattr(L, name).restype = ctypes.c_int
    _LIB = L
    return L


def check(fn: str, rc: int):
    if rc != 0:
        raise FkError(fn, rc)
