"""MI355X (gfx950) low-rank decoder-block hot path.

Python binding of liblrblock.so. The functions here only marshal torch
tensors into the C ABI of include/lr_block.h (device pointers, sizes and the
current HIP stream); every step of the block runs in the library's kernels.
Torch supplies device memory and streams. If the library has not been built
the first call raises; there is no other implementation to fall back on.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import (  # noqa: F401
    LR_BF16, LR_EPI_ADD_RESIDUAL, LR_EPI_NONE, LR_EPI_ROW_SCALE, LR_EPI_SWIGLU_PAIR, LR_F32,
    LR_LAYOUT_NN, LR_LAYOUT_NT, LR_LAYOUT_TN, LR_STAGE_ALL, LR_STAGE_POST_ATTN,
    LR_STAGE_PRE_ATTN, LR_WS_H, LR_WS_M, LRError, lr_block_shape,
)

WEIGHT_FIELDS = ("gamma1", "gamma2", "A_qkv", "B_q", "B_k", "B_v", "A_o", "B_o",
                 "A_gu", "B_g", "B_u", "A_dn", "B_dn")
SAVED_FIELDS = ("qkv_r", "o_r", "gu_r", "d_r", "rms1", "rms2")
PARTIAL_FIELDS = ("P_qkv", "P_gu", "ss1", "ss2")

_TORCH = {LR_F32: torch.float32, LR_BF16: torch.bfloat16}


def torch_dtype(dtype: int) -> torch.dtype:
    return _TORCH[dtype]


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("tensor is not on a GPU")
    if not t.is_contiguous():
        raise ValueError("tensor is not contiguous")
    return t.data_ptr()


def _stream(stream, device=None) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def block_shape(T, d, r, d_ff, d_norm=None, n_panels=1, n_heads=1, eps=1e-5, dtype=LR_BF16,
                emit_partials=False) -> lr_block_shape:
    return lr_block_shape(T=T, d=d, r=r, d_ff=d_ff, d_norm=d_norm or d, n_panels=n_panels,
                          n_heads=n_heads, eps=eps, dtype=dtype,
                          emit_partials=int(bool(emit_partials)))


def workspace_bytes(shape: lr_block_shape, is_bwd: bool) -> int:
    return int(_lib.load().lr_block_workspace_bytes(ctypes.byref(shape), int(bool(is_bwd))))


def workspace_tensor(shape: lr_block_shape, ws: torch.Tensor, is_bwd: bool, which: int):
    """View of the d-wide intermediate `which` (LR_WS_H or LR_WS_M) inside a
    block workspace (lr_block_workspace_tensor), as a [T, width] tensor."""
    off, nb = ctypes.c_size_t(), ctypes.c_size_t()
    _lib.check(_lib.load().lr_block_workspace_tensor(ctypes.byref(shape), int(bool(is_bwd)),
                                                     int(which), ctypes.byref(off),
                                                     ctypes.byref(nb)))
    dt = torch_dtype(shape.dtype)
    width = shape.d if which == _lib.LR_WS_H else shape.d_ff
    raw = ws[off.value:off.value + nb.value]
    return raw.view(dt).view(shape.T, width)


def alloc_workspace(shape: lr_block_shape, is_bwd: bool, device="cuda") -> torch.Tensor:
    n = workspace_bytes(shape, is_bwd)
    if n == 0:
        raise ValueError("invalid block shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _struct(cls, fields, d):
    s = cls()
    if d is not None:
        for f in fields:
            setattr(s, f, _ptr(d.get(f)))
    return s


def block_fwd(shape, W, X, O, out, saved, partials=None, stage=LR_STAGE_ALL, ws=None,
              stream=None) -> None:
    """lr_block_fwd. W, out (Q, K, V, Y), saved, partials: dicts of tensors."""
    lib = _lib.load()
    w = _struct(_lib.lr_block_weights, WEIGHT_FIELDS, W)
    sv = _struct(_lib.lr_block_saved, SAVED_FIELDS, saved)
    pt = _struct(_lib.lr_block_partials, PARTIAL_FIELDS, partials) if partials else None
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _lib.check(lib.lr_block_fwd(
        ctypes.byref(shape), ctypes.byref(w), _ptr(X), _ptr(O), _ptr(out.get("Q")),
        _ptr(out.get("K")), _ptr(out.get("V")), _ptr(out.get("Y")), ctypes.byref(sv),
        ctypes.byref(pt) if pt is not None else None, stage, _ptr(ws), nbytes,
        _stream(stream, X.device)))


def block_bwd(shape, W, X, O, saved, dY, dQ, dK, dV, dX, dO, grads, stage=LR_STAGE_ALL,
              ws=None, stream=None) -> None:
    """lr_block_bwd. grads: dict of fp32 tensors keyed like the weights."""
    lib = _lib.load()
    w = _struct(_lib.lr_block_weights, WEIGHT_FIELDS, W)
    sv = _struct(_lib.lr_block_saved, SAVED_FIELDS, saved)
    g = _struct(_lib.lr_block_grads, WEIGHT_FIELDS, grads)
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _lib.check(lib.lr_block_bwd(
        ctypes.byref(shape), ctypes.byref(w), _ptr(X), _ptr(O), ctypes.byref(sv), _ptr(dY),
        _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(dX), _ptr(dO), ctypes.byref(g), stage, _ptr(ws),
        nbytes, _stream(stream, X.device)))


def _pair_array(pairs, layout):
    arr = (_lib.lr_gemm_pair * len(pairs))()
    dev = None
    for i, p in enumerate(pairs):
        M, N, K = p["M"], p["N"], p["K"]
        ldx = p.get("ldx", M if layout == LR_LAYOUT_TN else K)
        ldw = p.get("ldw", K if layout == LR_LAYOUT_NT else N)
        aux = p.get("aux")
        arr[i] = _lib.lr_gemm_pair(M, N, K, _ptr(p["X"]), ldx, _ptr(p["W"]), ldw, _ptr(p["Y"]),
                                   p.get("ldy", N), _ptr(aux), p.get("ldaux", N))
        dev = p["X"].device
    return arr, dev


def grouped_lowrank_gemm(pairs, dtype, layout=LR_LAYOUT_NT, epilogue=LR_EPI_NONE,
                         stream=None, ws=None) -> None:
    """lr_grouped_lowrank_gemm (lr_grouped_lowrank_gemm_ws when a workspace
    tensor is given). pairs: list of dicts with M, N, K, X, W, Y, optional
    ldx, ldw, ldy (default: the contiguous row lengths), aux, ldaux."""
    lib = _lib.load()
    arr, dev = _pair_array(pairs, layout)
    if ws is None:
        _lib.check(lib.lr_grouped_lowrank_gemm(len(pairs), arr, dtype, layout, epilogue,
                                               _stream(stream, dev)))
    else:
        _lib.check(lib.lr_grouped_lowrank_gemm_ws(len(pairs), arr, dtype, layout, epilogue,
                                                  _ptr(ws), ws.numel() * ws.element_size(),
                                                  _stream(stream, dev)))


def grouped_lowrank_gemm_workspace_bytes(pairs, dtype, layout) -> int:
    """lr_grouped_lowrank_gemm_workspace_bytes for these pairs."""
    lib = _lib.load()
    arr, _ = _pair_array(pairs, layout)
    return int(lib.lr_grouped_lowrank_gemm_workspace_bytes(len(pairs), arr, dtype, layout))


def online_rmsnorm_gemm(X, gamma, A, out, *, n_panels=1, d_norm=None, eps=1e-5, rms_out=None,
                        ss_out=None, emit_partial=False, ws=None, stream=None) -> None:
    """lr_online_rmsnorm_gemm with contiguous X [T, d], A [N, d], out [T, N]."""
    lib = _lib.load()
    T, d = X.shape
    N = A.shape[0]
    dtype = LR_F32 if X.dtype == torch.float32 else LR_BF16
    if gamma is not None and ws is None:
        ws = torch.empty(int(lib.lr_online_rmsnorm_gemm_workspace_bytes(N, d, dtype)),
                         dtype=torch.uint8, device=X.device)
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    _lib.check(lib.lr_online_rmsnorm_gemm(
        T, d, N, n_panels, d_norm or d, eps, _ptr(X), d, _ptr(gamma), _ptr(A), d, _ptr(out), N,
        _ptr(rms_out), _ptr(ss_out), int(bool(emit_partial)), dtype, _ptr(ws), nbytes,
        _stream(stream, X.device)))


def online_rmsnorm_gemm_noalloc(X, gamma, A, out, *, n_panels=1, d_norm=None, eps=1e-5,
                                rms_out=None, ss_out=None, emit_partial=False,
                                stream=None) -> None:
    """lr_online_rmsnorm_gemm_noalloc: as online_rmsnorm_gemm, with the
    library's built-in scratch instead of a workspace."""
    lib = _lib.load()
    T, d = X.shape
    N = A.shape[0]
    dtype = LR_F32 if X.dtype == torch.float32 else LR_BF16
    _lib.check(lib.lr_online_rmsnorm_gemm_noalloc(
        T, d, N, n_panels, d_norm or d, eps, _ptr(X), d, _ptr(gamma), _ptr(A), d, _ptr(out), N,
        _ptr(rms_out), _ptr(ss_out), int(bool(emit_partial)), dtype, _stream(stream, X.device)))


def attn_shape(T, seq_len, n_heads, n_kv_heads=None, head_dim=128, rope_base=10000.0,
               dtype=LR_BF16) -> _lib.lr_attn_shape:
    return _lib.lr_attn_shape(T, seq_len, n_heads, n_kv_heads or n_heads, head_dim, dtype,
                              rope_base)


def attention_workspace_bytes(shape: _lib.lr_attn_shape, is_bwd: bool) -> int:
    return int(_lib.load().lr_attention_workspace_bytes(ctypes.byref(shape), int(bool(is_bwd))))


def _attn_ws(shape, is_bwd, ws, device):
    if ws is None:
        ws = torch.empty(max(attention_workspace_bytes(shape, is_bwd), 1), dtype=torch.uint8,
                         device=device)
    return ws, ws.numel() * ws.element_size()


def attention_fwd(shape, Q, K, V, O, lse, ws=None, stream=None) -> None:
    """lr_attention_fwd: O [T, H*128] and lse [H, T] (fp32) from Q, K, V."""
    lib = _lib.load()
    ws, nbytes = _attn_ws(shape, False, ws, Q.device)
    _lib.check(lib.lr_attention_fwd(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                    _ptr(lse), _ptr(ws), nbytes, _stream(stream, Q.device)))


def attention_bwd(shape, Q, K, V, O, dO, lse, dQ, dK, dV, ws=None, stream=None) -> None:
    """lr_attention_bwd: dQ, dK, dV from Q, K, V, the forward's O and lse, and dO."""
    lib = _lib.load()
    ws, nbytes = _attn_ws(shape, True, ws, Q.device)
    _lib.check(lib.lr_attention_bwd(ctypes.byref(shape), _ptr(Q), _ptr(K), _ptr(V), _ptr(O),
                                    _ptr(dO), _ptr(lse), _ptr(dQ), _ptr(dK), _ptr(dV), _ptr(ws),
                                    nbytes, _stream(stream, Q.device)))


def profile_enable(on: bool = True) -> None:
    """Start (True) or stop (False) per-kernel HIP-event timing in the library."""
    _lib.check(_lib.load().lr_profile_enable(int(bool(on))))


def profile_repeat(n: int) -> None:
    """While recording, enqueue each memory-bound launch n times between its events."""
    _lib.check(_lib.load().lr_profile_repeat(int(n)))


def profile_collect(max_kernels: int = 64, with_bytes: bool = False) -> list[tuple]:
    """Wait for the recorded events; return [(kernel, launches, total ms)], with
    ``with_bytes`` [(kernel, launches, total ms, algorithmic HBM bytes)]."""
    lib = _lib.load()
    arr = (_lib.lr_kernel_time * max_kernels)()
    n = lib.lr_profile_collect(arr, max_kernels)
    if n < 0:
        _lib.check(n)
    return [(arr[i].name.decode(), int(arr[i].count), float(arr[i].total_ms))
            + ((float(arr[i].bytes),) if with_bytes else ())
            for i in range(min(n, max_kernels))]


def version() -> str:
    return _lib.load().lr_version().decode()
