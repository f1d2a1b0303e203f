"""ctypes wrapper around the plain-C oracle (cider_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding.  It shares
no code with the HIP path.  Arrays are numpy; fp16 tensors travel as numpy
float16 (or their uint16 bit patterns).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "cider_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-Wall"]


def compile_oracle(src: str, out: str) -> str:
    """Compile an oracle C source into a shared library (host gcc only)."""
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = False) -> str:
    if force or not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < os.path.getmtime(SOURCE):
        compile_oracle(SOURCE, LIBRARY)
    return LIBRARY


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _half_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of fp16 values (or of bf16 values already given as
    uint16 patterns)."""
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    assert x.dtype == np.uint16, x.dtype
    return np.ascontiguousarray(x)


class OracleError(RuntimeError):
    pass


class Oracle:
    """One loaded oracle library (the real one, or a mutated copy in tests)."""

    def __init__(self, path: str | None = None):
        self.path = path or build()
        L = self.lib = ctypes.CDLL(self.path)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_half_to_double.restype = ctypes.c_double
        L.oracle_double_to_half.argtypes = [ctypes.c_double]
        L.oracle_double_to_half.restype = ctypes.c_uint16
        L.oracle_quantize_act.argtypes = [P, I64, I64, I64, P, P]
        L.oracle_quantize_weight.argtypes = [P, I64, I64, I, I, P, P]
        L.oracle_quantize_weight_clipped.argtypes = [P, I64, I64, I, I, ctypes.c_double, P, P]
        L.oracle_percentile_abs.argtypes = [P, I64, ctypes.c_double, P]
        L.oracle_percentile_abs.restype = ctypes.c_double
        D = ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = D
        L.oracle_double_to_bf16.argtypes = [D]
        L.oracle_double_to_bf16.restype = ctypes.c_uint16
        L.oracle_quantize_act_ex.argtypes = [P, I, I64, I64, I64, P, P, P]
        L.oracle_quantize_weight_ex.argtypes = [P, I, I64, I64, I, I, D, P, P]
        L.oracle_smooth_fold_weight.argtypes = [P, I, I64, I64, P, P]
        L.oracle_dequant_ex.argtypes = [P, P, P, I64, I64, I64, I, P]
        L.oracle_linear_ex.argtypes = [P, I, I64, I64, I64, P, P, P, I, I64, I, I, P, P, P]
        L.oracle_decode_linear.argtypes = [P, I, I64, P, P, I, I64, I, I, P]
        L.oracle_gemm_acc.argtypes = [P, P, I, I64, I64, I64, I, P]
        L.oracle_dequant.argtypes = [P, P, P, I64, I64, I64, P]
        L.oracle_linear.argtypes = [P, I64, I64, I64, P, P, I, I64, I, P, P, P]
        L.oracle_set_num_threads.argtypes = [I]
        L.oracle_set_num_threads.restype = None
        for f in ("oracle_quantize_act", "oracle_quantize_weight", "oracle_gemm_acc",
                  "oracle_dequant", "oracle_linear", "oracle_num_threads",
                  "oracle_quantize_weight_clipped", "oracle_quantize_act_ex",
                  "oracle_quantize_weight_ex", "oracle_smooth_fold_weight", "oracle_dequant_ex",
                  "oracle_linear_ex", "oracle_decode_linear"):
            getattr(L, f).restype = ctypes.c_int

    @staticmethod
    def _check(rc: int, what: str):
        if rc != 0:
            raise OracleError("oracle %s failed with code %d" % (what, rc))

    def num_threads(self) -> int:
        return self.lib.oracle_num_threads()

    def set_num_threads(self, n: int):
        """Thread count of later calls (scheduling only; results unchanged)."""
        self.lib.oracle_set_num_threads(int(n))

    def half_to_double(self, h: int) -> float:
        return self.lib.oracle_half_to_double(int(h))

    def double_to_half(self, v: float) -> int:
        return self.lib.oracle_double_to_half(float(v))

    def bf16_to_double(self, h: int) -> float:
        return self.lib.oracle_bf16_to_double(int(h))

    def double_to_bf16(self, v: float) -> int:
        return self.lib.oracle_double_to_bf16(float(v))

    @staticmethod
    def _smooth(smooth):
        if smooth is None:
            return None, None
        a = np.ascontiguousarray(smooth, dtype=np.float32)
        return a, _ptr(a)

    def quantize_act_ex(self, xbits: np.ndarray, dtype: int, K: int | None = None, smooth=None):
        """xbits: uint16 patterns [M, ldx] of fp16 (dtype 0) or bf16 (dtype 1)
        values; smooth: optional fp32 [K] divisors.  Returns (xq, s_tok)."""
        xb = _half_bits(xbits)
        M, ldx = xb.shape
        K = ldx if K is None else K
        sm, sp = self._smooth(smooth)
        xq = np.empty((M, K), np.int8)
        s = np.empty((M,), np.float32)
        self._check(self.lib.oracle_quantize_act_ex(_ptr(xb), dtype, M, K, ldx, sp, _ptr(xq),
                                                    _ptr(s)), "quantize_act_ex")
        return xq, s

    def quantize_weight_ex(self, wbits: np.ndarray, dtype: int, bits: int = 8,
                           group_size: int = 0, clip_percentile: float = 100.0):
        wb = _half_bits(wbits)
        N, K = wb.shape
        G = 1 if group_size == 0 else K // group_size
        wq = np.empty((N, K) if bits == 8 else (N, K // 2), np.int8 if bits == 8 else np.uint8)
        s = np.empty((N,) if group_size == 0 else (N, G), np.float32)
        self._check(self.lib.oracle_quantize_weight_ex(_ptr(wb), dtype, N, K, bits, group_size,
                                                       float(clip_percentile), _ptr(wq), _ptr(s)),
                    "quantize_weight_ex")
        return wq, s

    def smooth_fold_weight(self, wbits: np.ndarray, dtype: int, smooth) -> np.ndarray:
        """w * smooth[k], rounded once to the weight's type; uint16 patterns."""
        wb = _half_bits(wbits)
        N, K = wb.shape
        sm, sp = self._smooth(smooth)
        out = np.empty((N, K), np.uint16)
        self._check(self.lib.oracle_smooth_fold_weight(_ptr(wb), dtype, N, K, sp, _ptr(out)),
                    "smooth_fold_weight")
        return out

    def dequant_ex(self, acc: np.ndarray, s_tok: np.ndarray, s_w: np.ndarray, y_dtype: int):
        """uint16 patterns [M, N] of the fp16 / bf16 outputs."""
        a = acc if acc.ndim == 3 else acc[:, :, None]
        a = np.ascontiguousarray(a, dtype=np.int32)
        M, N, G = a.shape
        st = np.ascontiguousarray(s_tok, dtype=np.float32)
        sw = np.ascontiguousarray(np.asarray(s_w, dtype=np.float32).reshape(N, G))
        y = np.empty((M, N), np.uint16)
        self._check(self.lib.oracle_dequant_ex(_ptr(a), _ptr(st), _ptr(sw), M, N, G, y_dtype,
                                               _ptr(y)), "dequant_ex")
        return y

    def linear_ex(self, xbits: np.ndarray, x_dtype: int, wq: np.ndarray, s_w: np.ndarray,
                  bits: int = 8, group_size: int = 0, K: int | None = None, smooth=None,
                  y_dtype: int = 0):
        """Whole path; returns (y uint16 patterns [M, N], xq, s_tok)."""
        xb = _half_bits(xbits)
        M, ldx = xb.shape
        K = ldx if K is None else K
        N = wq.shape[0]
        wq = np.ascontiguousarray(wq)
        sw = np.ascontiguousarray(s_w, dtype=np.float32)
        sm, sp = self._smooth(smooth)
        xq = np.empty((M, K), np.int8)
        st = np.empty((M,), np.float32)
        y = np.empty((M, N), np.uint16)
        self._check(self.lib.oracle_linear_ex(_ptr(xb), x_dtype, M, K, ldx, sp, _ptr(wq), _ptr(sw),
                                              bits, N, group_size, y_dtype, _ptr(xq), _ptr(st),
                                              _ptr(y)), "linear_ex")
        return y, xq, st

    def decode_linear(self, xbits: np.ndarray, x_dtype: int, wq: np.ndarray, s_w: np.ndarray,
                      bits: int = 8, group_size: int = 0, y_dtype: int = 0) -> np.ndarray:
        """The decode variant: fp16 / bf16 x [K] against dequantized weights,
        no activation quantization.  Returns uint16 patterns [N]."""
        xb = _half_bits(np.ascontiguousarray(xbits).reshape(-1))
        K = xb.size
        wq = np.ascontiguousarray(wq)
        N = wq.shape[0]
        sw = np.ascontiguousarray(s_w, dtype=np.float32)
        y = np.empty((N,), np.uint16)
        self._check(self.lib.oracle_decode_linear(_ptr(xb), x_dtype, K, _ptr(wq), _ptr(sw), bits, N,
                                                  group_size, y_dtype, _ptr(y)), "decode_linear")
        return y

    def quantize_act(self, x: np.ndarray, K: int | None = None):
        """x: fp16 [M, ldx]; quantizes the first K (default: all) columns of
        every row.  Returns (xq int8 [M, K], s_tok fp32 [M])."""
        xb = _half_bits(x)
        M, ldx = xb.shape
        K = ldx if K is None else K
        xq = np.empty((M, K), np.int8)
        s = np.empty((M,), np.float32)
        self._check(self.lib.oracle_quantize_act(_ptr(xb), M, K, ldx, _ptr(xq), _ptr(s)),
                    "quantize_act")
        return xq, s

    def quantize_weight(self, w: np.ndarray, bits: int = 8, group_size: int = 0):
        """w: fp16 [N, K].  Returns (wq, s_w): int8 [N, K] (bits 8) or uint8
        [N, K/2] packed (bits 4); s_w fp32 [N] or [N, K/group_size]."""
        wb = _half_bits(w)
        N, K = wb.shape
        G = 1 if group_size == 0 else K // group_size
        if bits == 8:
            wq = np.empty((N, K), np.int8)
        else:
            wq = np.empty((N, K // 2), np.uint8)
        s = np.empty((N,) if group_size == 0 else (N, G), np.float32)
        self._check(self.lib.oracle_quantize_weight(_ptr(wb), N, K, bits, group_size,
                                                    _ptr(wq), _ptr(s)), "quantize_weight")
        return wq, s

    def quantize_weight_clipped(self, w: np.ndarray, bits: int, group_size: int,
                                clip_percentile: float):
        """As quantize_weight, with each row's (group's) range the
        clip_percentile-th percentile of its |w| instead of its absmax."""
        wb = _half_bits(w)
        N, K = wb.shape
        G = 1 if group_size == 0 else K // group_size
        wq = np.empty((N, K) if bits == 8 else (N, K // 2), np.int8 if bits == 8 else np.uint8)
        s = np.empty((N,) if group_size == 0 else (N, G), np.float32)
        self._check(self.lib.oracle_quantize_weight_clipped(
            _ptr(wb), N, K, bits, group_size, float(clip_percentile), _ptr(wq), _ptr(s)),
            "quantize_weight_clipped")
        return wq, s

    def percentile_abs(self, x: np.ndarray, p: float) -> float:
        """The p-th percentile of |x| (fp16 values) as the clipping uses it."""
        xb = _half_bits(np.ascontiguousarray(x).reshape(-1))
        buf = np.empty(xb.size, np.float64)
        return float(self.lib.oracle_percentile_abs(_ptr(xb), xb.size, float(p), _ptr(buf)))

    def gemm_acc(self, xq: np.ndarray, wq: np.ndarray, bits: int = 8,
                 group_size: int = 0) -> np.ndarray:
        """Integer accumulators: int32 [M, N] (group_size 0) or [M, N, K/gs]."""
        xq = np.ascontiguousarray(xq, dtype=np.int8)
        wq = np.ascontiguousarray(wq)
        M, K = xq.shape
        N = wq.shape[0]
        G = 1 if group_size == 0 else K // group_size
        acc = np.empty((M, N, G), np.int32)
        self._check(self.lib.oracle_gemm_acc(_ptr(xq), _ptr(wq), bits, M, N, K, group_size,
                                             _ptr(acc)), "gemm_acc")
        return acc[:, :, 0].copy() if group_size == 0 else acc

    def dequant(self, acc: np.ndarray, s_tok: np.ndarray, s_w: np.ndarray) -> np.ndarray:
        """fp16 [M, N] from acc [M, N] (per-channel) or [M, N, G] (per-group)."""
        a = acc if acc.ndim == 3 else acc[:, :, None]
        a = np.ascontiguousarray(a, dtype=np.int32)
        M, N, G = a.shape
        st = np.ascontiguousarray(s_tok, dtype=np.float32)
        sw = np.ascontiguousarray(np.asarray(s_w, dtype=np.float32).reshape(N, G))
        y = np.empty((M, N), np.uint16)
        self._check(self.lib.oracle_dequant(_ptr(a), _ptr(st), _ptr(sw), M, N, G, _ptr(y)),
                    "dequant")
        return y.view(np.float16)

    def linear(self, x: np.ndarray, wq: np.ndarray, s_w: np.ndarray, bits: int = 8,
               group_size: int = 0, K: int | None = None):
        """Whole path on fp16 x [M, ldx] (first K columns).
        Returns (y fp16 [M, N], xq int8 [M, K], s_tok fp32 [M])."""
        xb = _half_bits(x)
        M, ldx = xb.shape
        K = ldx if K is None else K
        N = wq.shape[0]
        wq = np.ascontiguousarray(wq)
        sw = np.ascontiguousarray(s_w, dtype=np.float32)
        xq = np.empty((M, K), np.int8)
        st = np.empty((M,), np.float32)
        y = np.empty((M, N), np.uint16)
        self._check(self.lib.oracle_linear(_ptr(xb), M, K, ldx, _ptr(wq), _ptr(sw), bits, N,
                                           group_size, _ptr(xq), _ptr(st), _ptr(y)), "linear")
        return y.view(np.float16), xq, st


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from cider_oracle.c."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
