"""The C-ABI library on the CPU: it loads, exports every entry point that
include/larosa.h declares, and rejects invalid arguments before touching a
device. Nothing here launches a kernel. Pointers below are fake addresses
that the library must never dereference (it checks arguments on the host
and returns before any HIP call)."""
import ctypes
import os
import re

import pytest

from rotated_top_activation_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "larosa.h")

OK, INVALID, SHAPE, ALIGN, DTYPE, WS, NODEV, LAUNCH, NONFINITE, TIMEOUT, INTERNAL = range(11)
P = 0x10000          # a fake, 16-byte aligned device address
PM = 0x10008         # a fake, misaligned one


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(larosa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from rotated_top_activation_amd import build
        build.build()
    return _lib.load()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"{n} has no binding"
    assert set(_lib.SIGNATURES) == set(names)


def test_version_and_status_strings(lib):
    assert lib.larosa_abi_version() == _lib.ABI_VERSION
    for code in range(11):
        assert lib.larosa_status_string(code) != b"unknown status"
    assert lib.larosa_status_string(99) == b"unknown status"


def test_workspace_bytes(lib):
    f = lib.larosa_workspace_bytes
    assert f(1, 4096, 22016, 2457, 0) > 0
    assert f(1, 4096, 22016, 0, 0) == 0          # k out of range
    assert f(1, 4096, 22016, 4097, 0) == 0
    assert f(1, 40000, 128, 10, 0) == 0          # d above 32768
    assert f(1, 4096, 22016, 2457, 8) == 0       # unknown mode bit
    assert f(1, 4096, 22016, 2457, 9) == 0
    # the fp64-rotation and validate flags need no extra workspace
    assert f(1, 4096, 22016, 2457, 2) == f(1, 4096, 22016, 2457, 0)
    assert f(1, 4096, 22016, 2457, 4) == f(1, 4096, 22016, 2457, 0)
    assert f(1, 4096, 22016, 2457, 7) == f(1, 4096, 22016, 2457, 1)
    assert f(4, 4096, 22016, 2457, 3) == f(4, 4096, 22016, 2457, 1)
    assert f(8, 4096, 22016, 2457, 0) >= f(1, 4096, 22016, 2457, 0)


def test_mlp_workspace_bytes(lib):
    m = lib.larosa_mlp_workspace_bytes
    args = (1, 4096, 11008, 2457, 6604)
    unf = m(*args, 0)
    assert unf > 0
    # the chained form takes the unfused layout; any mode's workspace holds
    # the one-launch up region, so the down region sits at one offset
    assert m(*args, 8) == unf
    assert m(*args, 8 | 2) == unf
    assert m(*args, 1) >= unf
    assert unf >= (lib.larosa_swiglu_workspace_bytes(1, 4096, 11008, 2457, 1) +
                   lib.larosa_workspace_bytes(1, 11008, 4096, 6604, 0))
    assert m(*args, 16) == 0          # unknown mode bit
    assert m(*args, 9 | 16) == 0


def _lf(lib, x=P, act=1, qt=P, qb=64, wf=P, wdt=1, B=1, d_in=128, d_out=64, k=32, y=P,
        idx=None, xr=None, mode=0, ws=P, wsb=1 << 30):
    return lib.larosa_layer_forward(x, act, qt, qb, wf, wdt, B, d_in, d_out, k, y, idx, xr,
                                    mode, ws, wsb, None)


def test_layer_forward_validation(lib):
    assert _lf(lib, k=0) == INVALID
    assert _lf(lib, k=129) == INVALID
    assert _lf(lib, B=-1) == INVALID
    assert _lf(lib, B=65) == INVALID
    assert _lf(lib, mode=8) == INVALID
    assert _lf(lib, mode=12) == INVALID
    assert _lf(lib, mode=2, k=0) == INVALID      # the flags do not skip the checks
    assert _lf(lib, mode=4, k=0) == INVALID
    assert _lf(lib, x=None) == INVALID
    assert _lf(lib, y=None) == INVALID
    assert _lf(lib, qb=48) == SHAPE             # does not divide 128
    assert _lf(lib, d_in=40000, k=10) == SHAPE
    assert _lf(lib, d_in=130, qb=130, k=10) == ALIGN   # d % 4
    assert _lf(lib, d_out=60) == ALIGN          # bf16 rows of 60 are not 16-byte units
    assert _lf(lib, x=PM) == ALIGN
    assert _lf(lib, wf=PM) == ALIGN
    assert _lf(lib, act=5) == DTYPE
    assert _lf(lib, act=1, wdt=0) == DTYPE      # bf16 activations need bf16 weights
    assert _lf(lib, ws=None) == WS
    assert _lf(lib, wsb=16) == WS
    assert _lf(lib, B=0) == OK                   # empty batch: nothing to do


def _qkv(lib, x=P, H=2, Hkv=1, dh=16, pos=5, theta=10000.0, B=1, k=32, ws=P, wsb=1 << 30,
         mode=0):
    # d_in 128, d_out (H + 2·Hkv)·dh
    return lib.larosa_qkv_rope_layer_forward(x, 1, P, 64, P, 1, B, 128, k, H, Hkv, dh, pos,
                                             ctypes.c_float(theta), P, None, None, mode, ws,
                                             wsb, None)


def test_qkv_rope_layer_validation(lib):
    assert _qkv(lib, H=0) == INVALID
    assert _qkv(lib, Hkv=0) == INVALID
    assert _qkv(lib, pos=-1) == INVALID
    assert _qkv(lib, theta=0.0) == INVALID
    assert _qkv(lib, theta=float("nan")) == INVALID
    assert _qkv(lib, dh=15) == SHAPE
    assert _qkv(lib, dh=0) == SHAPE
    assert _qkv(lib, dh=258) == SHAPE           # above 256
    assert _qkv(lib, k=0) == INVALID            # the layer's own checks follow
    assert _qkv(lib, x=PM) == ALIGN
    assert _qkv(lib, ws=None) == WS
    assert _qkv(lib, mode=9) == INVALID
    assert _qkv(lib, B=0) == OK


def test_standalone_calls_validation(lib):
    assert lib.larosa_rotate(P, 1, P, 48, 1, P, 1, 128, None) == SHAPE
    assert lib.larosa_rotate(P, 9, P, 64, 1, P, 1, 128, None) == DTYPE
    assert lib.larosa_rotate(None, 1, P, 64, 1, P, 1, 128, None) == INVALID
    assert lib.larosa_rotate(P, 1, P, 64, 1, PM, 1, 128, None) == ALIGN
    assert lib.larosa_rotate_fp64(P, 1, P, 48, 1, P, 1, 128, None) == SHAPE
    assert lib.larosa_rotate_fp64(P, 1, P, 64, 3, P, 1, 128, None) == DTYPE
    assert lib.larosa_rotate_fp64(P, 1, None, 64, 1, P, 1, 128, None) == INVALID
    assert lib.larosa_rotate_fp64(P, 1, P, 64, 1, P, 65, 128, None) == INVALID
    assert lib.larosa_rotate_fp64(PM, 1, P, 64, 1, P, 1, 128, None) == ALIGN
    assert lib.larosa_rotate_fp64(P, 1, P, 60, 1, P, 1, 120, None) == ALIGN  # d % 8, bf16
    assert lib.larosa_rotate_fp64(P, 1, P, 64, 1, P, 0, 128, None) == OK     # empty batch
    assert lib.larosa_swiglu_layer_forward(P, 1, P, 64, P, 1, 1, 128, 256, 10, P, None, None, 9,
                                           P, 1 << 24, None) == INVALID
    assert lib.larosa_topk_select(P, 1, 128, 0, P, P, None, None, None, None, None, 0,
                                  None) == INVALID
    assert lib.larosa_topk_select(P, 2, 128, 5, P, P, P, P, None, P, P, 1 << 20,
                                  None) == INVALID   # union without its count
    assert lib.larosa_topk_select(P, 2, 128, 5, P, P, P, P, P, P, P, 4, None) == WS
    assert lib.larosa_sparse_gemv(P, None, 10, P, P, 1, P, 1, 1, 128, 60, P, 1 << 20,
                                  None) == ALIGN
    assert lib.larosa_sparse_gemv(P, None, 10, P, P, 0, P, 1, 1, 128, 64, P, 1 << 20,
                                  None) == DTYPE     # fp32 weights into bf16 output
    assert lib.larosa_sparse_gemv(P, None, -1, P, P, 1, P, 1, 1, 128, 64, P, 1 << 20,
                                  None) == INVALID
    assert lib.larosa_dense_gemv(P, 1, P, 0, P, 1, 128, 64, P, 1 << 20, None) == DTYPE
    # selection folded into the product (one token)
    assert lib.larosa_topk_gemv(P, 128, 0, P, 1, P, 1, 64, None, P, 1 << 20, None) == INVALID
    assert lib.larosa_topk_gemv(P, 128, 129, P, 1, P, 1, 64, None, P, 1 << 20, None) == INVALID
    assert lib.larosa_topk_gemv(P, 20000, 10, P, 1, P, 1, 64, None, P, 1 << 20, None) == SHAPE
    assert lib.larosa_topk_gemv(P, 128, 10, P, 0, P, 1, 64, None, P, 1 << 20, None) == DTYPE
    assert lib.larosa_topk_gemv(P, 128, 10, P, 1, P, 1, 60, None, P, 1 << 20, None) == ALIGN
    assert lib.larosa_topk_gemv(PM, 128, 10, P, 1, P, 1, 64, None, P, 1 << 20, None) == ALIGN
    assert lib.larosa_topk_gemv(P, 128, 10, P, 1, P, 1, 64, None, P, 16, None) == WS
    assert lib.larosa_topk_gemv(None, 128, 10, P, 1, P, 1, 64, None, P, 1 << 20, None) == INVALID
    assert lib.larosa_fold_weights(P, 64, P, P, 128, 64, 1, None) == INVALID   # aliasing
    assert lib.larosa_prepare_rotation(P, P + 16, 128, 64, 1, None) == INVALID  # overlap
    assert lib.larosa_prepare_rotation(P, P + (1 << 20), 128, 48, 1, None) == SHAPE
    assert lib.larosa_swiglu(P, P, 1, 12, 1, None) == ALIGN
    assert lib.larosa_interleave_gate_up(P, P + (1 << 24), 64, 300, 1, None) == SHAPE
    assert lib.larosa_interleave_gate_up(P, P + 64, 64, 256, 1, None) == INVALID  # overlap
    assert lib.larosa_swiglu_workspace_bytes(1, 4096, 11008, 2457, 0) > \
        lib.larosa_workspace_bytes(1, 4096, 22016, 2457, 0)
    assert lib.larosa_swiglu_layer_forward(P, 1, P, 64, P, 1, 1, 128, 300, 10, P, None, None, 0,
                                           P, 1 << 24, None) == SHAPE
    assert lib.larosa_workspace_init(PM, 64, None) == ALIGN


def test_threshold_calls_validation(lib):
    nan = float("nan")
    ts = lib.larosa_threshold_select
    assert ts(P, 1, 128, -1.0, P, P, None, None, None, None, None, None, 0, None) == INVALID
    assert ts(P, 1, 128, nan, P, P, None, None, None, None, None, None, 0, None) == INVALID
    assert ts(P, 1, 128, 0.5, P, None, None, None, None, None, None, None, 0, None) == INVALID
    assert ts(P, 65, 128, 0.5, P, P, None, None, None, None, None, None, 0, None) == INVALID
    assert ts(P, 1, 40000, 0.5, P, P, None, None, None, None, None, None, 0, None) == SHAPE
    assert ts(P, 2, 128, 0.5, P, P, None, P, P, None, P, P, 1 << 20, None) == INVALID
    assert ts(P, 2, 128, 0.5, P, P, None, P, P, P, P, P, 4, None) == WS
    assert ts(PM, 1, 128, 0.5, P, P, None, None, None, None, None, None, 0, None) == ALIGN
    assert ts(P, 0, 128, 0.5, P, P, None, None, None, None, None, None, 0, None) == OK
    cw = lib.larosa_calibrate_workspace_bytes()
    assert 0 < cw < 1 << 16
    cal = lib.larosa_calibrate_threshold
    assert cal(P, 0, 1, P, P, cw, None) == SHAPE
    assert cal(P, 1 << 31, 1, P, P, cw, None) == SHAPE
    assert cal(P, 100, 0, P, P, cw, None) == INVALID
    assert cal(P, 100, 101, P, P, cw, None) == INVALID
    assert cal(P, 100, 10, None, P, cw, None) == INVALID
    assert cal(P, 100, 10, P, P, cw - 1, None) == WS
    assert cal(P, 100, 10, P, PM, cw, None) == ALIGN
    tl = lib.larosa_threshold_layer_forward
    args = (P, 1, P, 64, P, 1, 1, 128, 64)
    assert tl(*args, -0.5, P, None, None, None, 0, P, 1 << 30, None) == INVALID
    assert tl(*args, nan, P, None, None, None, 0, P, 1 << 30, None) == INVALID
    assert tl(*args, 0.5, P, None, None, None, 8, P, 1 << 30, None) == INVALID
    assert tl(*args, 0.5, P, None, None, None, 0, P, 16, None) == WS
    assert tl(P, 1, P, 48, P, 1, 1, 128, 64, 0.5, P, None, None, None, 0, P, 1 << 30,
              None) == SHAPE
    tsw = lib.larosa_threshold_swiglu_layer_forward
    assert tsw(P, 1, P, 64, P, 1, 1, 128, 256, -1.0, P, None, None, None, 0, P, 1 << 24,
               None) == INVALID
    assert tsw(P, 1, P, 64, P, 1, 1, 128, 300, 0.5, P, None, None, None, 0, P, 1 << 24,
               None) == SHAPE


def test_lowrank_validation(lib):
    wb = lib.larosa_lowrank_workspace_bytes
    assert wb(1, 4096, 22016, 2457, 64) > lib.larosa_workspace_bytes(1, 4096, 22016, 2457, 0)
    assert wb(1, 4096, 22016, 2457, 0) == 0       # r outside [1, 256]
    assert wb(1, 4096, 22016, 2457, 257) == 0
    assert wb(1, 128, 64, 10, 100) == 0           # r above d_out
    lr = lib.larosa_lowrank_layer_forward

    def call(r=16, a=P, wext=P, mode=0, wsb=1 << 30, k=32, qb=64):
        return lr(P, 1, P, qb, wext, a, r, 1, 1, 128, 64, k, P, None, None, mode, P, wsb, None)
    assert call(r=0) == INVALID
    assert call(r=65) == INVALID                  # above d_out = 64
    assert call(a=None) == INVALID
    assert call(wext=None) == INVALID
    assert call(mode=8) == INVALID
    assert call(k=0) == INVALID
    assert call(qb=48) == SHAPE
    assert call(wext=PM) == ALIGN
    assert call(wsb=16) == WS


def test_no_device_is_reported_not_crashed(lib):
    """Valid arguments on a machine without a GPU give NO_DEVICE."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert _lf(lib) == NODEV
    assert _lf(lib, mode=3) == NODEV
    assert lib.larosa_threshold_layer_forward(P, 1, P, 64, P, 1, 1, 128, 64, 0.5, P, None, None,
                                              None, 0, P, 1 << 30, None) == NODEV
    assert lib.larosa_calibrate_threshold(P, 100, 10, P, P, 1 << 16, None) == NODEV
    assert lib.larosa_lowrank_layer_forward(P, 1, P, 64, P, P, 16, 1, 1, 128, 64, 32, P, None,
                                            None, 0, P, 1 << 30, None) == NODEV
    assert lib.larosa_rotate_fp64(P, 1, P, 64, 1, P + (1 << 20), 1, 128, None) == NODEV
    assert lib.larosa_swiglu(P, P + (1 << 20), 1, 64, 1, None) == NODEV
    assert lib.larosa_topk_gemv(P, 128, 10, P, 1, P, 1, 64, None, P, 1 << 20, None) == NODEV
    assert _lf(lib, mode=_lib.VALIDATE) == NODEV
    assert lib.larosa_workspace_status(P, P + 256, None) == NODEV


def test_workspace_status_and_spin_limit_arguments(lib):
    st = lib.larosa_workspace_status
    assert st(None, P, None) == INVALID
    assert st(P, None, None) == INVALID
    assert st(PM, P, None) == ALIGN
    assert st(P, P + 2, None) == ALIGN           # status_out not 4-byte aligned
    prev = lib.larosa_set_spin_limit(7)
    assert prev == 1 << 22                       # the documented default
    assert lib.larosa_set_spin_limit(prev) == 7
    assert lib.larosa_set_spin_limit(prev) == prev


def test_entry_points_are_declared_no_throw():
    """Every declaration in the header carries the no-throw marker, and the
    C++ definitions repeat it (a mismatch would not compile)."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    decls = re.findall(r"\b(larosa_\w+)\s*\([^;]*\)\s*(LAROSA_NOEXCEPT)?\s*;", text)
    assert decls
    assert all(mark for _, mark in decls), [n for n, mark in decls if not mark]


def test_prerotated_flag_rules(lib):
    """LAROSA_PREROTATED (16): x is x_rot and Qt may be NULL; xrot_out must be
    NULL and the fp64 rotation flag cannot join it. Valid calls get past
    every argument check (to the device check, which fails here)."""
    assert _lf(lib, qt=None) == INVALID                 # a rotating call needs Qt
    assert _lf(lib, qt=None, mode=16) == NODEV
    assert _lf(lib, mode=16 | 1) == NODEV               # FUSED runs the unfused steps
    assert _lf(lib, mode=16, xr=P) == INVALID
    assert _lf(lib, mode=16 | 2) == INVALID
    assert _lf(lib, mode=16, k=0) == INVALID
    assert lib.larosa_workspace_bytes(1, 4096, 22016, 2457, 16) == \
        lib.larosa_workspace_bytes(1, 4096, 22016, 2457, 0)
    # the no-alloc call runs on x itself only
    na = lib.larosa_layer_forward_noalloc
    assert na(P, 1, P, 64, P, 1, 1, 128, 64, 32, P, None, None, 16, None) == INVALID
    assert na(P, 1, P, 64, P, 1, 1, 128, 64, 32, P, None, None, 0, None) == NODEV


def test_residual_rmsnorm_rotate_validation(lib):
    f = lib.larosa_residual_rmsnorm_rotate
    H, O, HO, A, Q, X = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000, 0x60000
    d = 4096
    assert f(H, O, HO, A, Q, d, 1e-5, X, 1, None) == NODEV     # every check passed
    assert f(H, None, None, None, Q, d, 1e-5, X, 1, None) == NODEV
    assert f(H, O, HO, A, Q, d, 1e-5, X, 0, None) == DTYPE      # bf16 only
    assert f(H, O, HO, A, Q, 256, 1e-5, X, 1, None) == SHAPE
    assert f(H, O, HO, A, Q, 8200, 1e-5, X, 1, None) == SHAPE
    assert f(H, O, HO, A, Q, 4100, 1e-5, X, 1, None) == SHAPE   # d % 8
    assert f(H, O, None, A, Q, d, 1e-5, X, 1, None) == INVALID  # o needs h_out
    assert f(H, O, H, A, Q, d, 1e-5, X, 1, None) == INVALID     # not in place
    assert f(H, O, H + 4096, A, Q, d, 1e-5, X, 1, None) == INVALID   # overlaps h
    assert f(H, O, HO, O, Q, d, 1e-5, X, 1, None) == INVALID    # a_out overlaps o
    assert f(H, O, HO, HO, Q, d, 1e-5, X, 1, None) == INVALID   # a_out overlaps h_out
    assert f(None, O, HO, A, Q, d, 1e-5, X, 1, None) == INVALID
    assert f(H, O, HO, A, None, d, 1e-5, X, 1, None) == INVALID
    assert f(H, O, HO, A, Q, d, -1.0, X, 1, None) == INVALID
    assert f(H + 8, O, HO, A, Q, d, 1e-5, X, 1, None) == ALIGN
    assert f(H, O, HO, A, Q, d, 1e-5, H + 4096, 1, None) == INVALID  # x_rot overlaps h
    assert f(H, O, HO, A, Q, d, 1e-5, O - 8192, 1, None) == INVALID  # x_rot (fp32) reaches o
    assert f(H, O, HO, A, Q, d, 1e-5, A - 16384, 1, None) == NODEV   # x_rot ends where a_out starts
    assert f(H, O, HO, A, Q, d, 1e-5, A - 16368, 1, None) == INVALID  # ... and one chunk more
