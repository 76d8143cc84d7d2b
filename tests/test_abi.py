"""The C ABI library loads, exports what include/lr_block.h declares, and
rejects bad arguments before touching the GPU (runs on hosts without one)."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

from gemm_online_rmsnorm_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lr_block.h")


def _ensure_built():
    if not os.path.exists(_lib.LIB_PATH):
        from gemm_online_rmsnorm_amd import build
        build.build()
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*(lr_[a-z0-9_]+)\s*\(",
                       text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_four_entry_points():
    names = _declared_functions()
    for n in ("lr_block_fwd", "lr_block_bwd", "lr_grouped_lowrank_gemm", "lr_online_rmsnorm_gemm"):
        assert n in names
    assert sorted(_lib.EXPORTS) == names


def test_library_exports_every_declared_symbol():
    lib = _ensure_built()
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(lr_[a-z0-9_]+)", out))
    for n in _declared_functions():
        assert n in exported, n
        assert hasattr(lib, n)


def _shape(**kw):
    base = dict(T=256, d=256, r=64, d_ff=688, d_norm=256, n_panels=1, n_heads=4, eps=1e-5,
                dtype=_lib.LR_F32, emit_partials=0)
    base.update(kw)
    return _lib.lr_block_shape(**base)


def _weights(addr=0x10000):
    w = _lib.lr_block_weights()
    for i, (f, _) in enumerate(_lib.lr_block_weights._fields_):
        setattr(w, f, addr + 0x100000 * i)
    return w


def _saved(addr=0x90000000):
    s = _lib.lr_block_saved()
    for i, (f, _) in enumerate(_lib.lr_block_saved._fields_):
        setattr(s, f, addr + 0x100000 * i)
    return s


def _fwd(lib, shape, w=None, ws=0xA0000000, ws_bytes=1 << 40, X=0x20000000, stage=0):
    w = w or _weights()
    sv = _saved()
    return lib.lr_block_fwd(ctypes.byref(shape), ctypes.byref(w), X, 0x30000000, 0x40000000,
                            0x50000000, 0x60000000, 0x70000000, ctypes.byref(sv), None, stage,
                            ws, ws_bytes, None)


def test_workspace_sizes():
    lib = _ensure_built()
    s = _shape()
    f = lib.lr_block_workspace_bytes(ctypes.byref(s), 0)
    b = lib.lr_block_workspace_bytes(ctypes.byref(s), 1)
    e = 4
    assert f >= e * (5 * 64 * 256 + 256 * 256 + 256 * 688)
    assert b >= e * (2 * 256 * 256 + 3 * 256 * 688 + 7 * 256 * 64)
    bad = _shape(d=250)
    assert lib.lr_block_workspace_bytes(ctypes.byref(bad), 0) == 0


@pytest.mark.parametrize("field,value,code", [
    ("T", 0, _lib.LR_ERR_INVALID_ARG),
    ("d", 250, _lib.LR_ERR_INVALID_ARG),          # not a multiple of the vector
    ("r", -4, _lib.LR_ERR_INVALID_ARG),
    ("dtype", 7, _lib.LR_ERR_INVALID_ARG),
    ("n_panels", 9, _lib.LR_ERR_INVALID_ARG),
    ("n_panels", 3, _lib.LR_ERR_INVALID_ARG),     # 256 does not split in 3
    ("n_panels", 8, _lib.LR_ERR_UNSUPPORTED),     # panels of 32 columns
    ("eps", float("nan"), _lib.LR_ERR_INVALID_ARG),
    ("emit_partials", 2, _lib.LR_ERR_INVALID_ARG),
])
def test_fwd_rejects_bad_shapes(field, value, code):
    lib = _ensure_built()
    s = _shape(**{field: value})
    assert _fwd(lib, s) == code
    assert lib.lr_last_error().decode() != ""


def test_fwd_rejects_null_and_misaligned_pointers_and_small_workspace():
    lib = _ensure_built()
    s = _shape()
    w = _weights()
    w.B_k = 0
    assert _fwd(lib, s, w=w) == _lib.LR_ERR_INVALID_ARG
    assert "B_k" in lib.lr_last_error().decode()
    w = _weights()
    w.A_o = 0x10008
    assert _fwd(lib, s, w=w) == _lib.LR_ERR_INVALID_ARG
    assert "aligned" in lib.lr_last_error().decode()
    assert _fwd(lib, s, X=0) == _lib.LR_ERR_INVALID_ARG
    assert _fwd(lib, s, ws_bytes=1024) == _lib.LR_ERR_WORKSPACE
    assert _fwd(lib, s, ws=0xA0000010) == _lib.LR_ERR_WORKSPACE
    assert _fwd(lib, s, stage=5) == _lib.LR_ERR_INVALID_ARG
    # rank-share mode needs the partials struct
    sp = _shape(emit_partials=1, d_norm=1024)
    assert _fwd(lib, sp) == _lib.LR_ERR_INVALID_ARG
    assert lib.lr_block_fwd(None, None, None, None, None, None, None, None, None, None, 0, None,
                            0, None) == _lib.LR_ERR_INVALID_ARG


def test_bwd_rejects_missing_grads():
    lib = _ensure_built()
    s = _shape()
    w, sv = _weights(), _saved()
    g = _lib.lr_block_grads()
    rc = lib.lr_block_bwd(ctypes.byref(s), ctypes.byref(w), 0x20000000, 0x30000000,
                          ctypes.byref(sv), 0x40000000, 0x50000000, 0x60000000, 0x70000000,
                          0x80000000, 0x88000000, ctypes.byref(g), 0, 0xA0000000, 1 << 40, None)
    assert rc == _lib.LR_ERR_INVALID_ARG
    assert lib.lr_block_bwd(ctypes.byref(s), ctypes.byref(w), 0x20000000, 0x30000000,
                            ctypes.byref(sv), 0, 0, 0, 0, 0, 0, None, 0, 0, 0, None) \
        == _lib.LR_ERR_INVALID_ARG


def test_grouped_gemm_validation():
    lib = _ensure_built()
    P = _lib.lr_gemm_pair
    good = P(64, 64, 64, 0x1000, 64, 0x2000, 64, 0x3000, 64, None, 0)
    arr = (P * 2)(good, good)
    assert lib.lr_grouped_lowrank_gemm(0, arr, _lib.LR_BF16, 0, 0, None) == _lib.LR_ERR_INVALID_ARG
    assert lib.lr_grouped_lowrank_gemm(4, arr, _lib.LR_BF16, 0, 0, None) == _lib.LR_ERR_INVALID_ARG
    assert lib.lr_grouped_lowrank_gemm(1, arr, _lib.LR_BF16, 9, 0, None) == _lib.LR_ERR_INVALID_ARG
    bad = (P * 1)(P(64, 64, 64, 0x1000, 60, 0x2000, 64, 0x3000, 64, None, 0))
    assert lib.lr_grouped_lowrank_gemm(1, bad, _lib.LR_BF16, 0, 0, None) == _lib.LR_ERR_INVALID_ARG
    # SwiGLU needs two pairs
    assert lib.lr_grouped_lowrank_gemm(1, arr, _lib.LR_BF16, 0, _lib.LR_EPI_SWIGLU_PAIR,
                                       None) == _lib.LR_ERR_UNSUPPORTED
    # unequal shapes in one call
    other = P(64, 32, 64, 0x1000, 64, 0x2000, 64, 0x3000, 64, None, 0)
    mixed = (P * 2)(good, other)
    assert lib.lr_grouped_lowrank_gemm(2, mixed, _lib.LR_BF16, 0, 0, None) == _lib.LR_ERR_UNSUPPORTED


def test_grouped_epilogue_inputs_are_per_pair_but_shared():
    """The epilogue's input (residual or row scale) travels in each pair; a
    grouped call must give every pair the same one, and the residual
    epilogue takes one pair."""
    lib = _ensure_built()
    P = _lib.lr_gemm_pair
    rs = lambda aux: P(64, 64, 64, 0x1000, 64, 0x2000, 64, 0x3000, 64, aux, 0)
    same = (P * 2)(rs(0x8000), rs(0x8000))
    diff = (P * 2)(rs(0x8000), rs(0x9000))
    f = lib.lr_grouped_lowrank_gemm
    assert f(2, diff, _lib.LR_BF16, _lib.LR_LAYOUT_NT, _lib.LR_EPI_ROW_SCALE, None) == \
        _lib.LR_ERR_UNSUPPORTED
    assert b"shared" in lib.lr_last_error()
    res = lambda: P(64, 64, 64, 0x1000, 64, 0x2000, 64, 0x3000, 64, 0x8000, 64)
    two = (P * 2)(res(), res())
    assert f(2, two, _lib.LR_BF16, _lib.LR_LAYOUT_NT, _lib.LR_EPI_ADD_RESIDUAL, None) == \
        _lib.LR_ERR_UNSUPPORTED
    # a missing row-scale input, and an epilogue on the TN layout
    assert f(1, (P * 1)(rs(None)), _lib.LR_BF16, _lib.LR_LAYOUT_NT, _lib.LR_EPI_ROW_SCALE,
             None) == _lib.LR_ERR_INVALID_ARG
    assert f(1, (P * 1)(rs(0x8000)), _lib.LR_BF16, _lib.LR_LAYOUT_TN, _lib.LR_EPI_ROW_SCALE,
             None) == _lib.LR_ERR_UNSUPPORTED
    assert same  # (a shared row scale is valid; it is run by the GPU tests)


def test_partials_struct_carries_the_two_norm_payloads():
    """The rank-share partials are the two Online RMSNorm payloads and their
    sums of squares; the other two chunks' payloads are o_r and d_r
    themselves (the saved activations)."""
    names = [f for f, _ in _lib.lr_block_partials._fields_]
    assert names == ["P_qkv", "P_gu", "ss1", "ss2"]
    text = open(HEADER).read()
    assert "P_o" not in re.sub(r"/\*.*?\*/", "", text, flags=re.S)


def test_grouped_gemm_workspace_variant_validation():
    """The workspace variant validates like the plain call and checks the
    workspace before launching anything (weight-gradient shape whose grid is
    too small to fill the GPU: K is split)."""
    lib = _ensure_built()
    P = _lib.lr_gemm_pair
    tn = (P * 1)(P(1024, 1024, 16384, 0x1000, 1024, 0x2000, 1024, 0x3000, 1024, None, 0))
    need = lib.lr_grouped_lowrank_gemm_workspace_bytes(1, tn, _lib.LR_BF16, _lib.LR_LAYOUT_TN)
    assert need > 0 and need % (1024 * 1024 * 4) == 0
    # fp32 and the other layouts need none
    assert lib.lr_grouped_lowrank_gemm_workspace_bytes(1, tn, _lib.LR_F32, _lib.LR_LAYOUT_TN) == 0
    nt = (P * 1)(P(64, 64, 64, 0x1000, 64, 0x2000, 64, 0x3000, 64, None, 0))
    assert lib.lr_grouped_lowrank_gemm_workspace_bytes(1, nt, _lib.LR_BF16, _lib.LR_LAYOUT_NT) == 0
    f = lib.lr_grouped_lowrank_gemm_ws
    assert f(0, tn, _lib.LR_BF16, _lib.LR_LAYOUT_TN, 0, 0x10000, need, None) == \
        _lib.LR_ERR_INVALID_ARG
    assert f(1, tn, _lib.LR_BF16, _lib.LR_LAYOUT_TN, 0, None, need, None) == _lib.LR_ERR_WORKSPACE
    assert f(1, tn, _lib.LR_BF16, _lib.LR_LAYOUT_TN, 0, 0x10010, need, None) == \
        _lib.LR_ERR_WORKSPACE
    assert f(1, tn, _lib.LR_BF16, _lib.LR_LAYOUT_TN, 0, 0x10000, need - 256, None) == \
        _lib.LR_ERR_WORKSPACE


def test_online_rmsnorm_gemm_validation():
    lib = _ensure_built()
    f = lib.lr_online_rmsnorm_gemm
    ok = dict(T=64, d=256, N=64, P=1, D=256, eps=1e-5, X=0x1000, ldx=256, g=0x2000, A=0x3000,
              lda=256, out=0x4000, ldo=64, rms=None, ss=None, part=0, dt=_lib.LR_BF16,
              ws=0x5000, wsb=1 << 30)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["T"], a["d"], a["N"], a["P"], a["D"], a["eps"], a["X"], a["ldx"], a["g"],
                 a["A"], a["lda"], a["out"], a["ldo"], a["rms"], a["ss"], a["part"], a["dt"],
                 a["ws"], a["wsb"], None)

    assert call(P=3) == _lib.LR_ERR_INVALID_ARG
    assert call(P=8) == _lib.LR_ERR_UNSUPPORTED
    assert call(wsb=16) == _lib.LR_ERR_WORKSPACE
    assert call(X=0x1001) == _lib.LR_ERR_INVALID_ARG
    assert call(ldx=100) == _lib.LR_ERR_INVALID_ARG
    assert call(part=3) == _lib.LR_ERR_INVALID_ARG
    assert lib.lr_online_rmsnorm_gemm_workspace_bytes(64, 256, _lib.LR_BF16) == 64 * 256 * 2


def test_profile_repeat_range():
    lib = _ensure_built()
    assert lib.lr_profile_repeat(0) == _lib.LR_ERR_INVALID_ARG
    assert b"out of range" in lib.lr_last_error()
    assert lib.lr_profile_repeat(1001) == _lib.LR_ERR_INVALID_ARG
    assert lib.lr_profile_repeat(20) == _lib.LR_OK
    assert lib.lr_profile_repeat(1) == _lib.LR_OK


def test_version_string():
    lib = _ensure_built()
    assert b"gfx950" in lib.lr_version()


def test_attention_validation():
    """The attention entry points reject unsupported or inconsistent shapes,
    bad pointers and short workspaces before launching anything."""
    lib = _ensure_built()
    S = _lib.lr_attn_shape

    def shape(**kw):
        d = dict(T=8192, seq_len=4096, n_heads=32, n_kv_heads=8, head_dim=128,
                 dtype=_lib.LR_BF16, rope_base=10000.0)
        d.update(kw)
        return S(**d)

    def nbytes(s, bwd):
        return lib.lr_attention_workspace_bytes(ctypes.byref(s), bwd)

    ok = shape()
    T, H, Hkv = 8192, 32, 8
    need_f, need_b = nbytes(ok, 0), nbytes(ok, 1)
    assert need_f >= T * (H + Hkv) * 128 * 2
    assert need_b >= need_f + T * H * 4
    fwd_args = (0x10000, 0x20000, 0x30000, 0x40000, 0x50000)

    def fwd(s, ws=0x100000, wsb=None):
        return lib.lr_attention_fwd(ctypes.byref(s), *fwd_args, ws,
                                    need_f if wsb is None else wsb, None)

    for kw, code in [(dict(seq_len=3000), _lib.LR_ERR_INVALID_ARG),   # T % seq_len
                     (dict(n_kv_heads=5), _lib.LR_ERR_INVALID_ARG),   # H % Hkv
                     (dict(n_heads=0), _lib.LR_ERR_INVALID_ARG),
                     (dict(head_dim=64), _lib.LR_ERR_UNSUPPORTED),
                     (dict(dtype=_lib.LR_F32), _lib.LR_ERR_UNSUPPORTED),
                     (dict(dtype=5), _lib.LR_ERR_INVALID_ARG),
                     (dict(rope_base=1.0), _lib.LR_ERR_INVALID_ARG),
                     (dict(rope_base=float("inf")), _lib.LR_ERR_INVALID_ARG),
                     (dict(T=1 << 20, seq_len=1 << 20, n_heads=64, n_kv_heads=8),
                      _lib.LR_ERR_UNSUPPORTED)]:                       # 32-bit offsets
        bad = shape(**kw)
        assert nbytes(bad, 0) == 0, kw
        assert fwd(bad) == code, kw
    assert fwd(ok, wsb=need_f - 1) == _lib.LR_ERR_WORKSPACE
    assert fwd(ok, ws=0x100008) == _lib.LR_ERR_WORKSPACE
    assert fwd(ok, ws=None) == _lib.LR_ERR_WORKSPACE
    assert lib.lr_attention_fwd(ctypes.byref(ok), 0x10008, 0x20000, 0x30000, 0x40000, 0x50000,
                                0x100000, need_f, None) == _lib.LR_ERR_INVALID_ARG
    assert lib.lr_attention_fwd(ctypes.byref(ok), 0x10000, 0x20000, 0x30000, 0x40000, 0x50002,
                                0x100000, need_f, None) == _lib.LR_ERR_INVALID_ARG
    bwd = lib.lr_attention_bwd
    ptrs = [0x10000 * (i + 1) for i in range(9)]
    assert bwd(ctypes.byref(ok), *ptrs, 0x100000, need_f, None) == _lib.LR_ERR_WORKSPACE
    ptrs[7] = 0  # dK
    assert bwd(ctypes.byref(ok), *ptrs, 0x100000, need_b, None) == _lib.LR_ERR_INVALID_ARG


def test_workspace_tensor_locations():
    """h and m lie inside their workspace, apart, with their sizes."""
    lib = _ensure_built()
    for dt, e in ((_lib.LR_F32, 4), (_lib.LR_BF16, 2)):
        s = _shape(dtype=dt)
        for is_bwd in (0, 1):
            total = lib.lr_block_workspace_bytes(ctypes.byref(s), is_bwd)
            spans = []
            for which, width in ((_lib.LR_WS_H, 256), (_lib.LR_WS_M, 688)):
                off, nb = ctypes.c_size_t(), ctypes.c_size_t()
                assert lib.lr_block_workspace_tensor(ctypes.byref(s), is_bwd, which,
                                                     ctypes.byref(off), ctypes.byref(nb)) == 0
                assert nb.value == e * 256 * width
                assert off.value % 256 == 0 and off.value + nb.value <= total
                spans.append((off.value, off.value + nb.value))
            (a0, a1), (b0, b1) = sorted(spans)
            assert a1 <= b0
    s = _shape()
    off, nb = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.lr_block_workspace_tensor(ctypes.byref(s), 0, 2, ctypes.byref(off),
                                         ctypes.byref(nb)) == _lib.LR_ERR_INVALID_ARG
    assert lib.lr_block_workspace_tensor(ctypes.byref(s), 0, 0, None, ctypes.byref(nb)) == \
        _lib.LR_ERR_INVALID_ARG
    bad = _shape(d=250)
    assert lib.lr_block_workspace_tensor(ctypes.byref(bad), 0, 0, ctypes.byref(off),
                                         ctypes.byref(nb)) == _lib.LR_ERR_INVALID_ARG


def test_online_rmsnorm_gemm_noalloc_validation():
    """The no-allocation variant checks like the workspace variant and
    rejects a gamma-folded A beyond its built-in scratch before any HIP
    call (these run on a host without a GPU)."""
    lib = _ensure_built()
    f = lib.lr_online_rmsnorm_gemm_noalloc
    cap = lib.lr_online_rmsnorm_gemm_noalloc_max_bytes()
    assert cap == 64 << 20
    ok = dict(T=64, d=256, N=64, P=1, D=256, eps=1e-5, X=0x1000, ldx=256, g=0x2000, A=0x3000,
              lda=256, out=0x4000, ldo=64, rms=None, ss=None, part=0, dt=_lib.LR_BF16)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["T"], a["d"], a["N"], a["P"], a["D"], a["eps"], a["X"], a["ldx"], a["g"],
                 a["A"], a["lda"], a["out"], a["ldo"], a["rms"], a["ss"], a["part"], a["dt"], None)

    assert call(P=3) == _lib.LR_ERR_INVALID_ARG
    assert call(P=8) == _lib.LR_ERR_UNSUPPORTED
    assert call(X=0x1001) == _lib.LR_ERR_INVALID_ARG
    assert call(part=3) == _lib.LR_ERR_INVALID_ARG
    # 8192 x 4104 bf16 is 64.1 MiB: one row past the scratch
    assert call(N=8192, d=4104, ldx=4104, lda=4104, ldo=8192) == _lib.LR_ERR_WORKSPACE
    assert b"scratch" in lib.lr_last_error()
    assert call(N=4096, d=4104, ldx=4104, lda=4104, ldo=4096, dt=_lib.LR_F32) == \
        _lib.LR_ERR_WORKSPACE
