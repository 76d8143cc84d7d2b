"""ctypes binding of liblrblock.so (the C ABI in include/lr_block.h).

Argument marshalling only: every step of the block runs in the library's HIP
kernels. Torch tensors supply device memory and the current HIP stream.
There is no fallback: if the library is missing the import of the binding
raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblrblock.so")

LR_OK = 0
LR_ERR_INVALID_ARG = -1
LR_ERR_UNSUPPORTED = -2
LR_ERR_WORKSPACE = -3
LR_ERR_HIP = -4

LR_F32, LR_BF16 = 0, 1
LR_STAGE_ALL, LR_STAGE_PRE_ATTN, LR_STAGE_POST_ATTN = 0, 1, 2
LR_LAYOUT_NT, LR_LAYOUT_NN, LR_LAYOUT_TN = 0, 1, 2
LR_EPI_NONE, LR_EPI_ADD_RESIDUAL, LR_EPI_SWIGLU_PAIR, LR_EPI_ROW_SCALE = 0, 1, 2, 3
LR_WS_H, LR_WS_M = 0, 1

# Every function include/lr_block.h declares.
EXPORTS = (
    "lr_block_workspace_bytes", "lr_block_workspace_tensor", "lr_block_fwd", "lr_block_bwd",
    "lr_grouped_lowrank_gemm", "lr_grouped_lowrank_gemm_workspace_bytes",
    "lr_grouped_lowrank_gemm_ws", "lr_online_rmsnorm_gemm_workspace_bytes",
    "lr_online_rmsnorm_gemm", "lr_online_rmsnorm_gemm_noalloc",
    "lr_online_rmsnorm_gemm_noalloc_max_bytes", "lr_attention_workspace_bytes", "lr_attention_fwd",
    "lr_attention_bwd", "lr_profile_enable", "lr_profile_collect", "lr_profile_repeat",
    "lr_last_error",
    "lr_version",
)


class lr_block_shape(ctypes.Structure):
    _fields_ = [("T", c_int64), ("d", c_int64), ("r", c_int64), ("d_ff", c_int64),
                ("d_norm", c_int64), ("n_panels", c_int32), ("n_heads", c_int32),
                ("eps", c_float), ("dtype", c_int32), ("emit_partials", c_int32)]


class lr_block_weights(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in (
        "gamma1", "gamma2", "A_qkv", "B_q", "B_k", "B_v", "A_o", "B_o",
        "A_gu", "B_g", "B_u", "A_dn", "B_dn")]


class lr_block_saved(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("qkv_r", "o_r", "gu_r", "d_r", "rms1", "rms2")]


class lr_block_grads(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in (
        "gamma1", "gamma2", "A_qkv", "B_q", "B_k", "B_v", "A_o", "B_o",
        "A_gu", "B_g", "B_u", "A_dn", "B_dn")]


class lr_block_partials(ctypes.Structure):
    _fields_ = [(n, c_void_p) for n in ("P_qkv", "P_gu", "ss1", "ss2")]


class lr_attn_shape(ctypes.Structure):
    _fields_ = [("T", c_int64), ("seq_len", c_int64), ("n_heads", c_int32),
                ("n_kv_heads", c_int32), ("head_dim", c_int32), ("dtype", c_int32),
                ("rope_base", ctypes.c_double)]


class lr_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("count", c_int32), ("total_ms", c_float),
                ("bytes", ctypes.c_double)]


class lr_gemm_pair(ctypes.Structure):
    _fields_ = [("M", c_int64), ("N", c_int64), ("K", c_int64), ("X", c_void_p),
                ("ldx", c_int64), ("W", c_void_p), ("ldw", c_int64), ("Y", c_void_p),
                ("ldy", c_int64), ("aux", c_void_p), ("ldaux", c_int64)]


_lib = None


def load(path: str | None = None):
    """Load the library (once). Raises OSError if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    p = path or os.environ.get("LRBLOCK_LIB", LIB_PATH)
    if not os.path.exists(p):
        raise OSError(f"liblrblock.so not found at {p}; run __graft_entry__.build() "
                      "(or python -m gemm_online_rmsnorm_amd.build) first")
    lib = ctypes.CDLL(p)
    S, W, SV, G, PT = (POINTER(lr_block_shape), POINTER(lr_block_weights),
                       POINTER(lr_block_saved), POINTER(lr_block_grads),
                       POINTER(lr_block_partials))
    lib.lr_block_workspace_bytes.argtypes = [S, c_int32]
    lib.lr_block_workspace_bytes.restype = c_size_t
    lib.lr_block_workspace_tensor.argtypes = [S, c_int32, c_int32, POINTER(c_size_t),
                                              POINTER(c_size_t)]
    lib.lr_block_workspace_tensor.restype = c_int32
    lib.lr_block_fwd.argtypes = [S, W, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                 c_void_p, SV, PT, c_int32, c_void_p, c_size_t, c_void_p]
    lib.lr_block_fwd.restype = c_int32
    lib.lr_block_bwd.argtypes = [S, W, c_void_p, c_void_p, SV, c_void_p, c_void_p, c_void_p,
                                 c_void_p, c_void_p, c_void_p, G, c_int32, c_void_p, c_size_t,
                                 c_void_p]
    lib.lr_block_bwd.restype = c_int32
    lib.lr_grouped_lowrank_gemm.argtypes = [c_int32, POINTER(lr_gemm_pair), c_int32, c_int32,
                                            c_int32, c_void_p]
    lib.lr_grouped_lowrank_gemm.restype = c_int32
    lib.lr_grouped_lowrank_gemm_workspace_bytes.argtypes = [c_int32, POINTER(lr_gemm_pair),
                                                            c_int32, c_int32]
    lib.lr_grouped_lowrank_gemm_workspace_bytes.restype = c_size_t
    lib.lr_grouped_lowrank_gemm_ws.argtypes = [c_int32, POINTER(lr_gemm_pair), c_int32, c_int32,
                                               c_int32, c_void_p, c_size_t, c_void_p]
    lib.lr_grouped_lowrank_gemm_ws.restype = c_int32
    lib.lr_online_rmsnorm_gemm_workspace_bytes.argtypes = [c_int64, c_int64, c_int32]
    lib.lr_online_rmsnorm_gemm_workspace_bytes.restype = c_size_t
    lib.lr_online_rmsnorm_gemm.argtypes = [
        c_int64, c_int64, c_int64, c_int32, c_int64, c_float, c_void_p, c_int64, c_void_p,
        c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_void_p, c_int32, c_int32, c_void_p,
        c_size_t, c_void_p]
    lib.lr_online_rmsnorm_gemm.restype = c_int32
    lib.lr_online_rmsnorm_gemm_noalloc.argtypes = [
        c_int64, c_int64, c_int64, c_int32, c_int64, c_float, c_void_p, c_int64, c_void_p,
        c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_void_p, c_int32, c_int32, c_void_p]
    lib.lr_online_rmsnorm_gemm_noalloc.restype = c_int32
    lib.lr_online_rmsnorm_gemm_noalloc_max_bytes.argtypes = []
    lib.lr_online_rmsnorm_gemm_noalloc_max_bytes.restype = c_size_t
    AS = POINTER(lr_attn_shape)
    lib.lr_attention_workspace_bytes.argtypes = [AS, c_int32]
    lib.lr_attention_workspace_bytes.restype = c_size_t
    lib.lr_attention_fwd.argtypes = [AS, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_size_t, c_void_p]
    lib.lr_attention_fwd.restype = c_int32
    lib.lr_attention_bwd.argtypes = [AS, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                     c_void_p]
    lib.lr_attention_bwd.restype = c_int32
    lib.lr_profile_enable.argtypes = [c_int32]
    lib.lr_profile_enable.restype = c_int32
    lib.lr_profile_collect.argtypes = [POINTER(lr_kernel_time), c_int32]
    lib.lr_profile_collect.restype = c_int32
    lib.lr_profile_repeat.argtypes = [c_int32]
    lib.lr_profile_repeat.restype = c_int32
    lib.lr_last_error.argtypes = []
    lib.lr_last_error.restype = ctypes.c_char_p
    lib.lr_version.argtypes = []
    lib.lr_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


class LRError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"lrblock error {code}: {msg}")
        self.code = code


def check(rc: int) -> None:
    if rc != LR_OK:
        raise LRError(rc, load().lr_last_error().decode())
