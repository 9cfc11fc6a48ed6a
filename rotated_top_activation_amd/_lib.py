"""ctypes binding of liblarosa.so — argument marshalling only.

Each ``larosa_*`` function here has the name and argument order of the C
entry point in ``include/larosa.h``. Tensor arguments are torch tensors on
the GPU (their ``data_ptr()`` is passed); dtypes are taken from the tensors;
``stream`` defaults to torch's current stream. A non-zero status raises
``LarosaError``. No step of the computation happens here.

The library must be built (``python -m rotated_top_activation_amd.build``);
importing a function does not load it, calling one does, and a missing
library raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblarosa.so")

F32, BF16 = 0, 1
UNFUSED, FUSED = 0, 1
ROTATE_FP64 = 2  # mode flag: fp64-accumulating rotation, OR-ed into UNFUSED or FUSED
VALIDATE = 4     # mode flag: check the rotated input for NaN/inf (waits on the stream)
CHAIN = 8        # mode flag of larosa_mlp_forward: the rotation of h chained into the gate|up launch
PREROTATED = 16  # mode flag of the layer calls: x is the rotated input x_rot (fp32)
ABI_VERSION = 9

# status codes (include/larosa.h)
OK, ERR_INVALID_ARG, ERR_SHAPE, ERR_ALIGNMENT, ERR_DTYPE, ERR_WORKSPACE = 0, 1, 2, 3, 4, 5
ERR_NO_DEVICE, ERR_LAUNCH, ERR_NONFINITE, ERR_TIMEOUT, ERR_INTERNAL = 6, 7, 8, 9, 10

_c_i64 = ctypes.c_int64
_c_int = ctypes.c_int
_c_vp = ctypes.c_void_p
_c_sz = ctypes.c_size_t

# (restype, argtypes) of every exported entry point.
SIGNATURES = {
    "larosa_abi_version": (_c_int, []),
    "larosa_status_string": (ctypes.c_char_p, [_c_int]),
    "larosa_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i64, _c_int]),
    "larosa_workspace_init": (_c_int, [_c_vp, _c_sz, _c_vp]),
    "larosa_workspace_status": (_c_int, [_c_vp, _c_vp, _c_vp]),
    "larosa_set_spin_limit": (ctypes.c_uint32, [ctypes.c_uint32]),
    "larosa_prepare_rotation": (_c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_int, _c_vp]),
    "larosa_fold_weights": (_c_int, [_c_vp, _c_i64, _c_vp, _c_vp, _c_i64, _c_i64, _c_int, _c_vp]),
    "larosa_rotate": (_c_int, [_c_vp, _c_int, _c_vp, _c_i64, _c_int, _c_vp, _c_i64, _c_i64, _c_vp]),
    "larosa_rotate_fp64": (_c_int, [_c_vp, _c_int, _c_vp, _c_i64, _c_int, _c_vp, _c_i64, _c_i64,
                                    _c_vp]),
    "larosa_topk_select": (_c_int, [_c_vp, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_vp,
                                    _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "larosa_sparse_gemv": (_c_int, [_c_vp, _c_vp, _c_i64, _c_vp, _c_vp, _c_int, _c_vp, _c_int,
                                    _c_i64, _c_i64, _c_i64, _c_vp, _c_sz, _c_vp]),
    "larosa_topk_gemv": (_c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_int, _c_vp, _c_int, _c_i64,
                                  _c_vp, _c_vp, _c_sz, _c_vp]),
    "larosa_layer_forward": (_c_int, [_c_vp, _c_int, _c_vp, _c_i64, _c_vp, _c_int, _c_i64,
                                      _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_int,
                                      _c_vp, _c_sz, _c_vp]),
    "larosa_layer_forward_noalloc": (_c_int, [_c_vp, _c_int, _c_vp, _c_i64, _c_vp, _c_int,
                                              _c_i64, _c_i64, _c_i64, _c_i64, _c_vp, _c_vp,
                                              _c_vp, _c_int, _c_vp]),
    "larosa_dense_gemv": (_c_int, [_c_vp, _c_int, _c_vp, _c_int, _c_vp, _c_i64, _c_i64, _c_i64,
                                   _c_vp, _c_sz, _c_vp]),
    "larosa_swiglu": (_c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_int, _c_vp]),
    "larosa_interleave_gate_up": (_c_int, [_c_vp, _c_vp, _c_i64, _c_i64, _c_int, _c_vp]),
    "larosa_swiglu_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i64, _c_int]),
    "larosa_swiglu_layer_forward": (_c_int, [_c_vp, _c_int, _c_vp, _c_i64, _c_vp, _c_int, _c_i64,
                                             _c_i64, _c_i64, _c_i64, _c_vp, _c_vp, _c_vp, _c_int,
                                             _c_vp, _c_sz, _c_vp]),
    "larosa_topk_swiglu_rotate": (_c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_int, _c_vp, _c_i64,
                                           _c_vp, _c_i64, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]),
    "larosa_mlp_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_int]),
    "larosa_mlp_forward": (_c_int, [_c_vp, _c_int, _c_vp, _c_i64, _c_vp, _c_vp, _c_i64, _c_vp,
                                    _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp,
                                    _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_int, _c_vp, _c_sz,
                                    _c_vp]),
    "larosa_calibrate_workspace_bytes": (_c_sz, []),
    "larosa_calibrate_threshold": (_c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_vp, _c_sz, _c_vp]),
    "larosa_threshold_select": (_c_int, [_c_vp, _c_i64, _c_i64, ctypes.c_float, _c_vp, _c_vp,
                                         _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz,
                                         _c_vp]),
    "larosa_threshold_layer_forward": (_c_int, [_c_vp, _c_int, _c_vp, _c_i64, _c_vp, _c_int,
                                                _c_i64, _c_i64, _c_i64, ctypes.c_float, _c_vp,
                                                _c_vp, _c_vp, _c_vp, _c_int, _c_vp, _c_sz,
                                                _c_vp]),
    "larosa_threshold_swiglu_layer_forward": (_c_int, [_c_vp, _c_int, _c_vp, _c_i64, _c_vp,
                                                       _c_int, _c_i64, _c_i64, _c_i64,
                                                       ctypes.c_float, _c_vp, _c_vp, _c_vp,
                                                       _c_vp, _c_int, _c_vp, _c_sz, _c_vp]),
    "larosa_lowrank_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64, _c_i64, _c_i64]),
    "larosa_lowrank_layer_forward": (_c_int, [_c_vp, _c_int, _c_vp, _c_i64, _c_vp, _c_vp, _c_i64,
                                              _c_int, _c_i64, _c_i64, _c_i64, _c_i64, _c_vp,
                                              _c_vp, _c_vp, _c_int, _c_vp, _c_sz, _c_vp]),
    "larosa_rmsnorm": (_c_int, [_c_vp, _c_vp, _c_i64, _c_i64, ctypes.c_float, _c_int, _c_vp]),
    "larosa_rope": (_c_int, [_c_vp, _c_i64, _c_vp, _c_vp, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                             ctypes.c_float, _c_int, _c_vp]),
    "larosa_qkv_rope_layer_forward": (_c_int, [_c_vp, _c_int, _c_vp, _c_i64, _c_vp, _c_int,
                                               _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_i64,
                                               _c_i64, ctypes.c_float, _c_vp, _c_vp, _c_vp,
                                               _c_int, _c_vp, _c_sz, _c_vp]),
    "larosa_decode_attention_workspace_bytes": (_c_sz, [_c_i64, _c_i64, _c_i64]),
    "larosa_decode_attention": (_c_int, [_c_vp, _c_vp, _c_i64, _c_vp, _c_i64, _c_vp, _c_vp, _c_vp,
                                         _c_i64, _c_i64, _c_i64, _c_i64, _c_i64, _c_int, _c_vp,
                                         _c_sz, _c_vp]),
    "larosa_residual_add": (_c_int, [_c_vp, _c_vp, _c_i64, _c_int, _c_vp]),
    "larosa_residual_rmsnorm": (_c_int, [_c_vp, _c_vp, _c_vp, _c_i64, _c_i64, ctypes.c_float,
                                         _c_int, _c_vp]),
    "larosa_residual_rmsnorm_rotate": (_c_int, [_c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_i64,
                                                ctypes.c_float, _c_vp, _c_int, _c_vp]),
    "larosa_topk_swiglu_gemv": (_c_int, [_c_vp, _c_i64, _c_i64, _c_vp, _c_int, _c_vp, _c_int,
                                         _c_i64, _c_vp, _c_vp, _c_sz, _c_vp]),
}

_lib = None


class LarosaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")


def load() -> ctypes.CDLL:
    """Load liblarosa.so once and declare its entry points."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m rotated_top_activation_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.larosa_abi_version() != ABI_VERSION:
            raise RuntimeError("liblarosa.so ABI version mismatch")
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().larosa_status_string(status).decode()


def _check(name: str, status: int) -> None:
    if status != 0:
        raise LarosaError(name, status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _act_dt(x, y, mode: int) -> int:
    """act_dtype of a layer call: y's type when x is the fp32 rotated input."""
    return _dt(y) if mode & PREROTATED else _dt(x)


def _dt(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(stream)
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _nbytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


# ----------------------------------------------------------------------------

def larosa_abi_version() -> int:
    return load().larosa_abi_version()


def larosa_workspace_bytes(B: int, d_in: int, d_out: int, k: int, mode: int = UNFUSED) -> int:
    return load().larosa_workspace_bytes(B, d_in, d_out, k, mode)


def larosa_workspace_init(ws, stream=None) -> None:
    _check("larosa_workspace_init",
           load().larosa_workspace_init(_ptr(ws), _nbytes(ws), _stream(stream)))


def larosa_workspace_status(ws, status_out, stream=None) -> None:
    _check("larosa_workspace_status",
           load().larosa_workspace_status(_ptr(ws), _ptr(status_out), _stream(stream)))


def larosa_set_spin_limit(limit: int) -> int:
    return int(load().larosa_set_spin_limit(limit))


def larosa_prepare_rotation(Q, Qt, d: int, q_block: int, stream=None) -> None:
    _check("larosa_prepare_rotation",
           load().larosa_prepare_rotation(_ptr(Q), _ptr(Qt), d, q_block, _dt(Q), _stream(stream)))


def larosa_fold_weights(Qt, q_block: int, W, W_folded, d_in: int, d_out: int,
                        stream=None) -> None:
    _check("larosa_fold_weights",
           load().larosa_fold_weights(_ptr(Qt), q_block, _ptr(W), _ptr(W_folded), d_in, d_out,
                                      _dt(W), _stream(stream)))


def larosa_rotate(x, Qt, q_block: int, x_rot, B: int, d: int, stream=None) -> None:
    _check("larosa_rotate",
           load().larosa_rotate(_ptr(x), _dt(x), _ptr(Qt), q_block, _dt(Qt), _ptr(x_rot), B, d,
                                _stream(stream)))


def larosa_rotate_fp64(x, Qt, q_block: int, x_rot, B: int, d: int, stream=None) -> None:
    _check("larosa_rotate_fp64",
           load().larosa_rotate_fp64(_ptr(x), _dt(x), _ptr(Qt), q_block, _dt(Qt), _ptr(x_rot), B,
                                     d, _stream(stream)))


def larosa_topk_select(x_rot, B: int, d: int, k: int, idx, val, xs=None, union_idx=None,
                       union_count=None, union_coef=None, ws=None, stream=None) -> None:
    _check("larosa_topk_select",
           load().larosa_topk_select(_ptr(x_rot), B, d, k, _ptr(idx), _ptr(val), _ptr(xs),
                                     _ptr(union_idx), _ptr(union_count), _ptr(union_coef),
                                     _ptr(ws), _nbytes(ws), _stream(stream)))


def larosa_sparse_gemv(rows, n_rows, max_rows: int, coef, W_folded, y, B: int, d_in: int,
                       d_out: int, ws=None, stream=None) -> None:
    _check("larosa_sparse_gemv",
           load().larosa_sparse_gemv(_ptr(rows), _ptr(n_rows), max_rows, _ptr(coef),
                                     _ptr(W_folded), _dt(W_folded), _ptr(y), _dt(y), B, d_in,
                                     d_out, _ptr(ws), _nbytes(ws), _stream(stream)))


def larosa_topk_gemv(x_rot, d_in: int, k: int, W_folded, y, d_out: int, idx_out=None, ws=None,
                     stream=None) -> None:
    _check("larosa_topk_gemv",
           load().larosa_topk_gemv(_ptr(x_rot), d_in, k, _ptr(W_folded), _dt(W_folded), _ptr(y),
                                   _dt(y), d_out, _ptr(idx_out), _ptr(ws), _nbytes(ws),
                                   _stream(stream)))


def larosa_layer_forward(x, Qt, q_block: int, W_folded, B: int, d_in: int, d_out: int, k: int,
                         y, idx_out=None, xrot_out=None, mode: int = UNFUSED, ws=None,
                         stream=None) -> None:
    _check("larosa_layer_forward",
           load().larosa_layer_forward(_ptr(x), _act_dt(x, y, mode), _ptr(Qt), q_block,
                                       _ptr(W_folded), _dt(W_folded), B, d_in, d_out, k, _ptr(y),
                                       _ptr(idx_out), _ptr(xrot_out), mode, _ptr(ws), _nbytes(ws),
                                       _stream(stream)))


def larosa_layer_forward_noalloc(x, Qt, q_block: int, W_folded, B: int, d_in: int, d_out: int,
                                 k: int, y, idx_out=None, xrot_out=None, mode: int = UNFUSED,
                                 stream=None) -> None:
    _check("larosa_layer_forward_noalloc",
           load().larosa_layer_forward_noalloc(_ptr(x), _act_dt(x, y, mode), _ptr(Qt), q_block,
                                               _ptr(W_folded), _dt(W_folded), B, d_in, d_out, k,
                                               _ptr(y), _ptr(idx_out), _ptr(xrot_out), mode,
                                               _stream(stream)))


def larosa_dense_gemv(x, W, y, B: int, d_in: int, d_out: int, ws=None, stream=None) -> None:
    _check("larosa_dense_gemv",
           load().larosa_dense_gemv(_ptr(x), _dt(x), _ptr(W), _dt(W), _ptr(y), B, d_in, d_out,
                                    _ptr(ws), _nbytes(ws), _stream(stream)))


def larosa_swiglu(gu, h, B: int, f: int, stream=None) -> None:
    _check("larosa_swiglu",
           load().larosa_swiglu(_ptr(gu), _ptr(h), B, f, _dt(gu), _stream(stream)))


def larosa_interleave_gate_up(W, W_il, d_in: int, f: int, stream=None) -> None:
    _check("larosa_interleave_gate_up",
           load().larosa_interleave_gate_up(_ptr(W), _ptr(W_il), d_in, f, _dt(W), _stream(stream)))


def larosa_swiglu_workspace_bytes(B: int, d_in: int, f: int, k: int, mode: int = UNFUSED) -> int:
    return int(load().larosa_swiglu_workspace_bytes(B, d_in, f, k, mode))


def larosa_swiglu_layer_forward(x, Qt, q_block: int, W_il, B: int, d_in: int, f: int, k: int,
                                h, idx_out=None, xrot_out=None, mode: int = UNFUSED, ws=None,
                                stream=None) -> None:
    _check("larosa_swiglu_layer_forward",
           load().larosa_swiglu_layer_forward(_ptr(x), _act_dt(x, h, mode), _ptr(Qt), q_block,
                                              _ptr(W_il), _dt(W_il), B, d_in, f, k, _ptr(h),
                                              _ptr(idx_out), _ptr(xrot_out), mode, _ptr(ws),
                                              _nbytes(ws), _stream(stream)))


def larosa_calibrate_workspace_bytes() -> int:
    return int(load().larosa_calibrate_workspace_bytes())


def larosa_calibrate_threshold(x_rot, n: int, keep: int, t_out, ws, stream=None) -> None:
    _check("larosa_calibrate_threshold",
           load().larosa_calibrate_threshold(_ptr(x_rot), n, keep, _ptr(t_out), _ptr(ws),
                                             _nbytes(ws), _stream(stream)))


def larosa_threshold_select(x_rot, B: int, d: int, t: float, idx, count, val=None, xs=None,
                            union_idx=None, union_count=None, union_coef=None, ws=None,
                            stream=None) -> None:
    _check("larosa_threshold_select",
           load().larosa_threshold_select(_ptr(x_rot), B, d, t, _ptr(idx), _ptr(count), _ptr(val),
                                          _ptr(xs), _ptr(union_idx), _ptr(union_count),
                                          _ptr(union_coef), _ptr(ws), _nbytes(ws),
                                          _stream(stream)))


def larosa_threshold_layer_forward(x, Qt, q_block: int, W_folded, B: int, d_in: int, d_out: int,
                                   t: float, y, idx_out=None, count_out=None, xrot_out=None,
                                   mode: int = UNFUSED, ws=None, stream=None) -> None:
    _check("larosa_threshold_layer_forward",
           load().larosa_threshold_layer_forward(_ptr(x), _dt(x), _ptr(Qt), q_block,
                                                 _ptr(W_folded), _dt(W_folded), B, d_in, d_out, t,
                                                 _ptr(y), _ptr(idx_out), _ptr(count_out),
                                                 _ptr(xrot_out), mode, _ptr(ws), _nbytes(ws),
                                                 _stream(stream)))


def larosa_threshold_swiglu_layer_forward(x, Qt, q_block: int, W_il, B: int, d_in: int, f: int,
                                          t: float, h, idx_out=None, count_out=None,
                                          xrot_out=None, mode: int = UNFUSED, ws=None,
                                          stream=None) -> None:
    _check("larosa_threshold_swiglu_layer_forward",
           load().larosa_threshold_swiglu_layer_forward(_ptr(x), _dt(x), _ptr(Qt), q_block,
                                                        _ptr(W_il), _dt(W_il), B, d_in, f, t,
                                                        _ptr(h), _ptr(idx_out), _ptr(count_out),
                                                        _ptr(xrot_out), mode, _ptr(ws),
                                                        _nbytes(ws), _stream(stream)))


def larosa_lowrank_workspace_bytes(B: int, d_in: int, d_out: int, k: int, r: int) -> int:
    return int(load().larosa_lowrank_workspace_bytes(B, d_in, d_out, k, r))


def larosa_lowrank_layer_forward(x, Qt, q_block: int, W_ext, A_r, r: int, B: int, d_in: int,
                                 d_out: int, k: int, y, idx_out=None, xrot_out=None,
                                 mode: int = UNFUSED, ws=None, stream=None) -> None:
    _check("larosa_lowrank_layer_forward",
           load().larosa_lowrank_layer_forward(_ptr(x), _dt(x), _ptr(Qt), q_block, _ptr(W_ext),
                                               _ptr(A_r), r, _dt(W_ext), B, d_in, d_out, k,
                                               _ptr(y), _ptr(idx_out), _ptr(xrot_out), mode,
                                               _ptr(ws), _nbytes(ws), _stream(stream)))


def larosa_rmsnorm(h, out, B: int, d: int, eps: float = 1e-5, stream=None) -> None:
    _check("larosa_rmsnorm", load().larosa_rmsnorm(_ptr(h), _ptr(out), B, d, eps, _dt(h),
                                                   _stream(stream)))


def larosa_rope(qk, qk_stride: int, q_out, k_out, B: int, n_heads: int, n_kv_heads: int,
                d_head: int, pos: int, theta: float = 10000.0, stream=None) -> None:
    _check("larosa_rope", load().larosa_rope(_ptr(qk), qk_stride, _ptr(q_out), _ptr(k_out), B,
                                             n_heads, n_kv_heads, d_head, pos, theta, _dt(qk),
                                             _stream(stream)))


def larosa_qkv_rope_layer_forward(x, Qt, q_block: int, W_folded, B: int, d_in: int, k: int,
                                  n_heads: int, n_kv_heads: int, d_head: int, pos: int, y,
                                  theta: float = 10000.0, idx_out=None, xrot_out=None,
                                  mode: int = UNFUSED, ws=None, stream=None) -> None:
    _check("larosa_qkv_rope_layer_forward",
           load().larosa_qkv_rope_layer_forward(_ptr(x), _act_dt(x, y, mode), _ptr(Qt), q_block,
                                                _ptr(W_folded), _dt(W_folded), B, d_in, k,
                                                n_heads, n_kv_heads, d_head, pos, theta, _ptr(y),
                                                _ptr(idx_out), _ptr(xrot_out), mode, _ptr(ws),
                                                _nbytes(ws), _stream(stream)))


def larosa_decode_attention_workspace_bytes(B: int, T: int, n_heads: int) -> int:
    return int(load().larosa_decode_attention_workspace_bytes(B, T, n_heads))


def larosa_decode_attention(q, k_new, k_stride: int, v_new, v_stride: int, k_cache, v_cache,
                            out, B: int, T: int, n_heads: int, n_kv_heads: int,
                            d_head: int = 128, ws=None, stream=None) -> None:
    _check("larosa_decode_attention",
           load().larosa_decode_attention(_ptr(q), _ptr(k_new), k_stride, _ptr(v_new), v_stride,
                                          _ptr(k_cache), _ptr(v_cache), _ptr(out), B, T, n_heads,
                                          n_kv_heads, d_head, _dt(q), _ptr(ws), _nbytes(ws),
                                          _stream(stream)))


def larosa_residual_add(h, o, n: int, stream=None) -> None:
    _check("larosa_residual_add", load().larosa_residual_add(_ptr(h), _ptr(o), n, _dt(h),
                                                             _stream(stream)))


def larosa_residual_rmsnorm_rotate(h, o, h_out, Qt, x_rot, d: int, a_out=None, eps: float = 1e-5,
                                   stream=None) -> None:
    _check("larosa_residual_rmsnorm_rotate",
           load().larosa_residual_rmsnorm_rotate(_ptr(h), _ptr(o), _ptr(h_out), _ptr(a_out),
                                                 _ptr(Qt), d, eps, _ptr(x_rot), _dt(h),
                                                 _stream(stream)))


def larosa_residual_rmsnorm(h, o, out, B: int, d: int, eps: float = 1e-5, stream=None) -> None:
    _check("larosa_residual_rmsnorm",
           load().larosa_residual_rmsnorm(_ptr(h), _ptr(o), _ptr(out), B, d, eps, _dt(h),
                                          _stream(stream)))


def larosa_topk_swiglu_gemv(x_rot, d_in: int, k: int, W_il, h, f: int, idx_out=None, ws=None,
                            stream=None) -> None:
    _check("larosa_topk_swiglu_gemv",
           load().larosa_topk_swiglu_gemv(_ptr(x_rot), d_in, k, _ptr(W_il), _dt(W_il), _ptr(h),
                                          _dt(h), f, _ptr(idx_out), _ptr(ws), _nbytes(ws),
                                          _stream(stream)))


def larosa_mlp_workspace_bytes(B: int, d: int, f: int, k1: int, k2: int,
                               mode: int = UNFUSED) -> int:
    return int(load().larosa_mlp_workspace_bytes(B, d, f, k1, k2, mode))


def larosa_mlp_forward(x, Qt1, q_block1: int, W_il, Qt2, q_block2: int, W_down, B: int, d: int,
                       f: int, k1: int, k2: int, h, y, idx1_out=None, xrot1_out=None,
                       idx2_out=None, xrot2_out=None, mode: int = UNFUSED, ws=None,
                       stream=None) -> None:
    _check("larosa_mlp_forward",
           load().larosa_mlp_forward(_ptr(x), _dt(x), _ptr(Qt1), q_block1, _ptr(W_il), _ptr(Qt2),
                                     q_block2, _ptr(W_down), _dt(W_il), B, d, f, k1, k2, _ptr(h),
                                     _ptr(y), _ptr(idx1_out), _ptr(xrot1_out), _ptr(idx2_out),
                                     _ptr(xrot2_out), mode, _ptr(ws), _nbytes(ws),
                                     _stream(stream)))


def larosa_topk_swiglu_rotate(x_rot, d_in: int, k: int, W_il, h, f: int, Qt2, q_block2: int,
                              x_rot2, idx_out=None, ws=None, stream=None) -> None:
    _check("larosa_topk_swiglu_rotate",
           load().larosa_topk_swiglu_rotate(_ptr(x_rot), d_in, k, _ptr(W_il), _dt(W_il), _ptr(h),
                                            f, _ptr(Qt2), q_block2, _ptr(x_rot2), _ptr(idx_out),
                                            _ptr(ws), _nbytes(ws), _stream(stream)))
