"""Python binding of libcider.so, the MI355X (gfx950) fused quantized linear
layer: per-token INT8 activation quantization, INT8 x INT8 -> INT32 product on
the matrix cores, fused dequantization to fp16 (W8A8 per channel, W8A8 per
group of 64 / 128, W4A8 with packed int4 weights).

This module only marshals arguments: every function has the name and the
argument order of the C function declared in include/cider.h, takes device
tensors (or raw integer device pointers) and a stream, and returns the
cider_status.  With ``check=True`` (the default) a non-zero status raises
CiderError.  All computation happens in the HIP kernels of libcider.so;
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_PKG, "libcider.so")

CIDER_OK = 0
CIDER_ERR_INVALID_ARG = 1
CIDER_ERR_UNSUPPORTED_SHAPE = 2
CIDER_ERR_MISALIGNED = 3
CIDER_ERR_NO_DEVICE = 4
CIDER_ERR_HIP = 5
CIDER_ERR_WORKSPACE = 6
CIDER_ERR_SCRATCH_LIMIT = 7
CIDER_NOALLOC_SCRATCH_BYTES = 64 << 20

PATH_AUTO, PATH_GEMV, PATH_GEMM = 0, 1, 2

EXPORTS = (
    "cider_is_available", "cider_status_str", "cider_quantize_weight", "cider_quantize_act",
    "cider_w8a8_gemm", "cider_w4a8_gemm", "cider_w8a8_gemm_i32", "cider_w4a8_gemm_i32",
    "cider_linear_workspace_bytes", "cider_linear_workspace_bytes_ex", "cider_w8a8_linear", "cider_w4a8_linear", "cider_set_path",
    "cider_quantize_weight_clipped", "cider_quantize_weight_ex", "cider_smooth_fold_weight",
    "cider_quantize_act_ex", "cider_gemm_ex", "cider_linear_ex", "cider_decode_linear",
    "cider_linear_ex_noalloc",
)

CIDER_DTYPE_F16 = 0
CIDER_DTYPE_BF16 = 1


class CiderError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (what, cider_status_str(status), status))


_lib: ctypes.CDLL | None = None


def load(build_if_missing: bool = True) -> ctypes.CDLL:
    """Load libcider.so.  When it has never been built, build it first (hipcc
    for gfx950); a load failure raises, there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIBRARY):
        if not build_if_missing:
            raise ImportError("libcider.so is not built (run __graft_entry__.build())")
        from . import build as _build
        _build.build(force=True)
    lib = ctypes.CDLL(LIBRARY)
    P, I64, I, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    sig = {
        "cider_is_available": ([], I),
        "cider_status_str": ([I], ctypes.c_char_p),
        "cider_quantize_weight": ([P, I64, I64, I, I, P, P, P], I),
        "cider_quantize_act": ([P, I64, I64, I64, P, P, P], I),
        "cider_quantize_weight_clipped": ([P, I64, I64, I, I, ctypes.c_double, P, P, P], I),
        "cider_quantize_weight_ex": ([P, I, I64, I64, I, I, ctypes.c_double, P, P, P], I),
        "cider_smooth_fold_weight": ([P, I, I64, I64, P, P, P], I),
        "cider_quantize_act_ex": ([P, I, I64, I64, I64, P, P, P, P], I),
        "cider_gemm_ex": ([P, P, P, P, I64, I64, I64, I, I, I, P, P], I),
        "cider_linear_ex": ([P, I, I64, I64, I64, P, P, P, I64, I, I, I, P, SZ, P, P], I),
        "cider_linear_ex_noalloc": ([P, I, I64, I64, I64, P, P, P, I64, I, I, I, P, P], I),
        "cider_decode_linear": ([P, I64, P, P, I64, I, I, I, P, P], I),
        "cider_w8a8_gemm": ([P, P, P, P, I64, I64, I64, I, P, P], I),
        "cider_w4a8_gemm": ([P, P, P, P, I64, I64, I64, I, P, P], I),
        "cider_w8a8_gemm_i32": ([P, P, I64, I64, I64, I, P, P], I),
        "cider_w4a8_gemm_i32": ([P, P, I64, I64, I64, I, P, P], I),
        "cider_linear_workspace_bytes": ([I64, I64], SZ),
        "cider_linear_workspace_bytes_ex": ([I64, I64, I64, I, I], SZ),
        "cider_w8a8_linear": ([P, I64, I64, I64, P, P, I64, I, P, SZ, P, P], I),
        "cider_w4a8_linear": ([P, I64, I64, I64, P, P, I64, I, P, SZ, P, P], I),
        "cider_set_path": ([I], I),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ret(status: int, what: str, check: bool) -> int:
    if check and status != CIDER_OK:
        raise CiderError(status, what)
    return status


def cider_is_available() -> bool:
    return bool(load().cider_is_available())


def cider_status_str(status: int) -> str:
    return load().cider_status_str(int(status)).decode()


def cider_quantize_weight(w_f16, N, K, bits, group_size, wq, s_w, stream=None, check=True):
    st = load().cider_quantize_weight(_ptr(w_f16), N, K, bits, group_size, _ptr(wq), _ptr(s_w),
                                      _stream(stream))
    return _ret(st, "cider_quantize_weight", check)


def cider_quantize_weight_clipped(w_f16, N, K, bits, group_size, clip_percentile, wq, s_w,
                                  stream=None, check=True):
    st = load().cider_quantize_weight_clipped(_ptr(w_f16), N, K, bits, group_size,
                                              float(clip_percentile), _ptr(wq), _ptr(s_w),
                                              _stream(stream))
    return _ret(st, "cider_quantize_weight_clipped", check)


def cider_quantize_weight_ex(w, w_dtype, N, K, bits, group_size, clip_percentile, wq, s_w,
                             stream=None, check=True):
    st = load().cider_quantize_weight_ex(_ptr(w), w_dtype, N, K, bits, group_size,
                                         float(clip_percentile), _ptr(wq), _ptr(s_w),
                                         _stream(stream))
    return _ret(st, "cider_quantize_weight_ex", check)


def cider_smooth_fold_weight(w, w_dtype, N, K, smooth, w_out, stream=None, check=True):
    st = load().cider_smooth_fold_weight(_ptr(w), w_dtype, N, K, _ptr(smooth), _ptr(w_out),
                                         _stream(stream))
    return _ret(st, "cider_smooth_fold_weight", check)


def cider_quantize_act_ex(x, x_dtype, M, K, ldx, smooth, xq, s_tok, stream=None, check=True):
    st = load().cider_quantize_act_ex(_ptr(x), x_dtype, M, K, ldx, _ptr(smooth), _ptr(xq),
                                      _ptr(s_tok), _stream(stream))
    return _ret(st, "cider_quantize_act_ex", check)


def cider_gemm_ex(xq, s_tok, wq, s_w, M, N, K, bits, group_size, y_dtype, y, stream=None,
                  check=True):
    st = load().cider_gemm_ex(_ptr(xq), _ptr(s_tok), _ptr(wq), _ptr(s_w), M, N, K, bits,
                              group_size, y_dtype, _ptr(y), _stream(stream))
    return _ret(st, "cider_gemm_ex", check)


def cider_linear_ex(x, x_dtype, M, K, ldx, smooth, wq, s_w, N, bits, group_size, y_dtype,
                    workspace, workspace_bytes, y, stream=None, check=True):
    st = load().cider_linear_ex(_ptr(x), x_dtype, M, K, ldx, _ptr(smooth), _ptr(wq), _ptr(s_w),
                                N, bits, group_size, y_dtype, _ptr(workspace), workspace_bytes,
                                _ptr(y), _stream(stream))
    return _ret(st, "cider_linear_ex", check)


def cider_linear_ex_noalloc(x, x_dtype, M, K, ldx, smooth, wq, s_w, N, bits, group_size, y_dtype,
                            y, stream=None, check=True):
    st = load().cider_linear_ex_noalloc(_ptr(x), x_dtype, M, K, ldx, _ptr(smooth), _ptr(wq),
                                        _ptr(s_w), N, bits, group_size, y_dtype, _ptr(y),
                                        _stream(stream))
    return _ret(st, "cider_linear_ex_noalloc", check)


def cider_decode_linear(x_f16, K, wq, s_w, N, bits, group_size, y_dtype, y, stream=None,
                        check=True):
    st = load().cider_decode_linear(_ptr(x_f16), K, _ptr(wq), _ptr(s_w), N, bits, group_size,
                                    y_dtype, _ptr(y), _stream(stream))
    return _ret(st, "cider_decode_linear", check)


def cider_quantize_act(x_f16, M, K, ldx, xq, s_tok, stream=None, check=True):
    st = load().cider_quantize_act(_ptr(x_f16), M, K, ldx, _ptr(xq), _ptr(s_tok), _stream(stream))
    return _ret(st, "cider_quantize_act", check)


def cider_w8a8_gemm(xq, s_tok, wq, s_w, M, N, K, group_size, y_f16, stream=None, check=True):
    st = load().cider_w8a8_gemm(_ptr(xq), _ptr(s_tok), _ptr(wq), _ptr(s_w), M, N, K, group_size,
                                _ptr(y_f16), _stream(stream))
    return _ret(st, "cider_w8a8_gemm", check)


def cider_w4a8_gemm(xq, s_tok, wq4, s_w, M, N, K, group_size, y_f16, stream=None, check=True):
    st = load().cider_w4a8_gemm(_ptr(xq), _ptr(s_tok), _ptr(wq4), _ptr(s_w), M, N, K, group_size,
                                _ptr(y_f16), _stream(stream))
    return _ret(st, "cider_w4a8_gemm", check)


def cider_w8a8_gemm_i32(xq, wq, M, N, K, group_size, acc, stream=None, check=True):
    st = load().cider_w8a8_gemm_i32(_ptr(xq), _ptr(wq), M, N, K, group_size, _ptr(acc),
                                    _stream(stream))
    return _ret(st, "cider_w8a8_gemm_i32", check)


def cider_w4a8_gemm_i32(xq, wq4, M, N, K, group_size, acc, stream=None, check=True):
    st = load().cider_w4a8_gemm_i32(_ptr(xq), _ptr(wq4), M, N, K, group_size, _ptr(acc),
                                    _stream(stream))
    return _ret(st, "cider_w4a8_gemm_i32", check)


def cider_linear_workspace_bytes(M, K) -> int:
    return int(load().cider_linear_workspace_bytes(M, K))


def cider_linear_workspace_bytes_ex(M, N, K, bits, group_size) -> int:
    return int(load().cider_linear_workspace_bytes_ex(M, N, K, bits, group_size))


def cider_w8a8_linear(x_f16, M, K, ldx, wq, s_w, N, group_size, workspace, workspace_bytes,
                      y_f16, stream=None, check=True):
    st = load().cider_w8a8_linear(_ptr(x_f16), M, K, ldx, _ptr(wq), _ptr(s_w), N, group_size,
                                  _ptr(workspace), workspace_bytes, _ptr(y_f16), _stream(stream))
    return _ret(st, "cider_w8a8_linear", check)


def cider_w4a8_linear(x_f16, M, K, ldx, wq4, s_w, N, group_size, workspace, workspace_bytes,
                      y_f16, stream=None, check=True):
    st = load().cider_w4a8_linear(_ptr(x_f16), M, K, ldx, _ptr(wq4), _ptr(s_w), N, group_size,
                                  _ptr(workspace), workspace_bytes, _ptr(y_f16), _stream(stream))
    return _ret(st, "cider_w4a8_linear", check)


def cider_set_path(path: int) -> int:
    return int(load().cider_set_path(int(path)))
