"""CPU oracle of the LLM.int8() mixed-precision decomposition matmul.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg use it.  The HIP library never imports, links or calls it,
and it shares no code with the HIP library.  The arithmetic lives in
``oracle.c`` (plain loops, fp32 scale arithmetic, exact integer sums, fp64
outlier sum, its own binary16 conversion); this module only moves numpy
arrays in and out of it.  ``brute.py`` is a second, pure-Python
implementation used to cross-check the C code on tiny shapes.

Pages followed (see oracle.c for the step-by-step definition):
  - lowentro.cn "model quantization" notes, Q2 (symmetric quantization
    formulas), Q3 (per-channel scales), Q4 (LLM.int8 decomposition), Q11
    (outliers; int8 range [-127, 127]);
  - hncyxsy.com/news/230290, section 2.1 (vector-wise quantization,
    threshold 6.0, fp16 outlier product, sum in fp16);
  - tqpw.cn/news/5683, section 2.1 (scale = max|W|/127, round, clip; worked
    example) and section 3.1 (LLM.int8 summary).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_u16p = ctypes.POINTER(ctypes.c_uint16)
_i8p = ctypes.POINTER(ctypes.c_int8)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64


def lib():
    """Load liboracle.so, compiling it first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or (
                os.path.getmtime(_LIB) < os.path.getmtime(os.path.join(_HERE, "oracle.c"))):
            from . import build as _b
            _b.build()
        L = ctypes.CDLL(_LIB)
        L.oracle_h2d.restype = ctypes.c_double
        L.oracle_h2d.argtypes = [ctypes.c_uint16]
        L.oracle_d2h.restype = ctypes.c_uint16
        L.oracle_d2h.argtypes = [ctypes.c_double]
        L.oracle_h2d_array.argtypes = [_u16p, _i64, _f64p]
        L.oracle_d2h_array.argtypes = [_f64p, _i64, _u16p]
        L.oracle_quantize_weight.argtypes = [_u16p, _i64, _i64, _i8p, _f32p]
        L.oracle_detect_outliers.argtypes = [_u16p, _i64, _i64, ctypes.c_double,
                                             _u8p, _i32p, _i32p]
        L.oracle_quantize_rows.argtypes = [_u16p, _i64, _i64, _u8p, _i8p, _f32p]
        L.oracle_int8_gemm.argtypes = [_i8p, _i8p, _i64, _i64, _i64, _i32p]
        L.oracle_decomposed_output.argtypes = [_u16p, _i32p, _f32p, _i8p, _f32p,
                                               _i32p, ctypes.c_int32,
                                               _i64, _i64, _i64, _u16p]
        L.oracle_decomposed_output_fp16w.argtypes = [_u16p, _i32p, _f32p, _f32p, _u16p,
                                                     _i32p, ctypes.c_int32,
                                                     _i64, _i64, _i64, _u16p]
        L.oracle_linear.restype = ctypes.c_int
        L.oracle_linear.argtypes = [_u16p, _i8p, _f32p, _u16p, ctypes.c_double,
                                    _i64, _i64, _i64, _u16p,
                                    _u8p, _i32p, _i32p, _i8p, _f32p, _i32p]
        L.oracle_sq_factors.argtypes = [_f32p, _f32p, ctypes.c_double, _i64, _f32p]
        L.oracle_column_absmax.argtypes = [_u16p, _i64, _i64, _f32p]
        L.oracle_sq_quantize_weight.argtypes = [_u16p, _f32p, _i64, _i64, _i8p, _f32p]
        L.oracle_sq_quantize_rows.argtypes = [_u16p, _f32p, _i64, _i64, _i8p, _f32p]
        L.oracle_sq_output.argtypes = [_i32p, _f32p, _f32p, _i64, _i64, _u16p]
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray, t):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(t)


def _f16bits(X) -> np.ndarray:
    X = np.ascontiguousarray(X)
    if X.dtype == np.float16:
        return X.view(np.uint16)
    assert X.dtype == np.uint16, X.dtype
    return X


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def h2d(bits: np.ndarray) -> np.ndarray:
    """Exact value of each binary16 bit pattern, as float64."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, np.float64)
    lib().oracle_h2d_array(_p(bits, _u16p), bits.size, _p(out, _f64p))
    return out


def d2h(x: np.ndarray) -> np.ndarray:
    """Round float64 values to binary16 (ties to even); returns the bits."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_d2h_array(_p(x, _f64p), x.size, _p(out, _u16p))
    return out


def quantize_weight(W):
    """Per-output-feature absmax int8 codes: (Wq int8 [N,K], sW fp32 [N])."""
    W = _f16bits(W)
    N, K = W.shape
    Wq = np.empty((N, K), np.int8)
    sW = np.empty(N, np.float32)
    lib().oracle_quantize_weight(_p(W, _u16p), N, K, _p(Wq, _i8p), _p(sW, _f32p))
    return Wq, sW


def detect_outliers(X, threshold: float):
    """(flags uint8 [K], idx int32 [nO] ascending) of columns with some |x| > thr."""
    X = _f16bits(X)
    T, K = X.shape
    flags = np.empty(K, np.uint8)
    idx = np.empty(max(K, 1), np.int32)
    nO = ctypes.c_int32(0)
    lib().oracle_detect_outliers(_p(X, _u16p), T, K, float(threshold),
                                 _p(flags, _u8p), ctypes.byref(nO), _p(idx, _i32p))
    return flags, idx[: nO.value].copy()


def quantize_rows(X, flags):
    """Token-wise codes over the normal columns: (Xq int8 [R,K], sX fp32 [R])."""
    X = _f16bits(X)
    R, K = X.shape
    flags = np.ascontiguousarray(flags, dtype=np.uint8)
    Xq = np.empty((R, K), np.int8)
    sX = np.empty(R, np.float32)
    lib().oracle_quantize_rows(_p(X, _u16p), R, K, _p(flags, _u8p), _p(Xq, _i8p), _p(sX, _f32p))
    return Xq, sX


def int8_gemm(Xq, Wq):
    """acc int32 [R,N] = Xq [R,K] . Wq[N,K]^T, exact."""
    Xq = np.ascontiguousarray(Xq, dtype=np.int8)
    Wq = np.ascontiguousarray(Wq, dtype=np.int8)
    R, K = Xq.shape
    N = Wq.shape[0]
    acc = np.empty((R, N), np.int32)
    lib().oracle_int8_gemm(_p(Xq, _i8p), _p(Wq, _i8p), R, N, K, _p(acc, _i32p))
    return acc


def decomposed_output(X, acc, sX, Wq, sW, idx, W16=None):
    """Y fp16 [R,N] from the int8 part (acc, sX, sW) and the outlier columns;
    with W16 (the fp16 weight [N,K]) the outlier columns use it instead of
    the dequantized codes."""
    X = _f16bits(X)
    R, K = X.shape
    N = Wq.shape[0]
    acc = np.ascontiguousarray(acc, dtype=np.int32)
    sX = np.ascontiguousarray(sX, dtype=np.float32)
    Wq = np.ascontiguousarray(Wq, dtype=np.int8)
    sW = np.ascontiguousarray(sW, dtype=np.float32)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    if idx.size == 0:
        idx = np.zeros(1, np.int32)
        nO = 0
    else:
        nO = len(idx)
    Y = np.empty((R, N), np.uint16)
    if W16 is None:
        lib().oracle_decomposed_output(_p(X, _u16p), _p(acc, _i32p), _p(sX, _f32p),
                                       _p(Wq, _i8p), _p(sW, _f32p), _p(idx, _i32p), nO,
                                       R, K, N, _p(Y, _u16p))
    else:
        W16 = _f16bits(W16)
        lib().oracle_decomposed_output_fp16w(_p(X, _u16p), _p(acc, _i32p), _p(sX, _f32p),
                                             _p(sW, _f32p), _p(W16, _u16p), _p(idx, _i32p), nO,
                                             R, K, N, _p(Y, _u16p))
    return Y.view(np.float16)


def linear(X, Wq, sW, threshold: float, stages: bool = False, W16=None):
    """The whole call.  Returns Y fp16 [T,N], or a dict with every stage.
    With W16 (the fp16 weight) the outlier columns use it (the fp16-weight
    variant)."""
    X = _f16bits(X)
    W16 = None if W16 is None else _f16bits(W16)
    T, K = X.shape
    Wq = np.ascontiguousarray(Wq, dtype=np.int8)
    sW = np.ascontiguousarray(sW, dtype=np.float32)
    N = Wq.shape[0]
    Y = np.empty((T, N), np.uint16)
    flags = np.empty(max(K, 1), np.uint8)
    idx = np.empty(max(K, 1), np.int32)
    Xq = np.empty((T, K), np.int8)
    sX = np.empty(max(T, 1), np.float32)
    acc = np.empty((T, N), np.int32)
    nO = ctypes.c_int32(0)
    w16p = None if W16 is None else _p(W16, _u16p)
    rc = lib().oracle_linear(_p(X, _u16p), _p(Wq, _i8p), _p(sW, _f32p), w16p, float(threshold),
                             T, K, N, _p(Y, _u16p), _p(flags, _u8p), ctypes.byref(nO),
                             _p(idx, _i32p), _p(Xq, _i8p), _p(sX, _f32p), _p(acc, _i32p))
    if rc != 0:
        raise MemoryError("oracle_linear failed to allocate")
    Y = Y.view(np.float16)
    if not stages:
        return Y
    return dict(Y=Y, flags=flags[:K].copy(), idx=idx[: nO.value].copy(), nO=nO.value,
                Xq=Xq, sX=sX[:T].copy(), acc=acc)


def linear_rows(X, Wq, sW, threshold: float, rows, W16=None):
    """Y for a subset of rows of a (possibly very large) call.

    The outlier set depends on every row of X, so detection runs over all
    of X; quantization, the int8 product and the output then run only for
    the requested rows.  Returns (Y_rows fp16 [len(rows), N], idx, Xq_rows,
    sX_rows, acc_rows).
    """
    X = _f16bits(X)
    flags, idx = detect_outliers(X, threshold)
    Xr = np.ascontiguousarray(X[np.asarray(rows)])
    Xq, sX = quantize_rows(Xr, flags)
    acc = int8_gemm(Xq, Wq)
    Y = decomposed_output(Xr, acc, sX, Wq, sW, idx, W16=W16)
    return Y, idx, Xq, sX, acc


# --------------------------------------------------------------------------
# SmoothQuant-style W8A8 (lowentro.cn notes, Q9-Q10; hncyxsy.com/news/230290, section 5.1): see oracle.c
# --------------------------------------------------------------------------

def column_absmax(X):
    """max_t |X[t,j]| per column, fp32 [K]."""
    X = _f16bits(X)
    R, K = X.shape
    out = np.empty(max(K, 1), np.float32)
    lib().oracle_column_absmax(_p(X, _u16p), R, K, _p(out, _f32p))
    return out[:K]


def sq_factors(ax, aw, alpha: float):
    """s_j = ax_j^alpha / aw_j^(1-alpha) in fp64, rounded to fp32 (1 where
    either maximum is 0)."""
    ax = np.ascontiguousarray(ax, dtype=np.float32)
    aw = np.ascontiguousarray(aw, dtype=np.float32)
    K = ax.shape[0]
    s = np.empty(max(K, 1), np.float32)
    lib().oracle_sq_factors(_p(ax, _f32p), _p(aw, _f32p), float(alpha), K, _p(s, _f32p))
    return s[:K]


def sq_quantize_weight(W, s):
    """(Wq int8 [N,K], sW fp32 [N]) of the smoothed weight W * s."""
    W = _f16bits(W)
    N, K = W.shape
    s = np.ascontiguousarray(s, dtype=np.float32)
    Wq = np.empty((N, K), np.int8)
    sW = np.empty(max(N, 1), np.float32)
    lib().oracle_sq_quantize_weight(_p(W, _u16p), _p(s, _f32p), N, K, _p(Wq, _i8p), _p(sW, _f32p))
    return Wq, sW[:N]


def sq_quantize_rows(X, s):
    """(Xq int8 [R,K], sX fp32 [R]) of the smoothed activation X * fl32(1/s)."""
    X = _f16bits(X)
    R, K = X.shape
    s = np.ascontiguousarray(s, dtype=np.float32)
    Xq = np.empty((R, K), np.int8)
    sX = np.empty(max(R, 1), np.float32)
    lib().oracle_sq_quantize_rows(_p(X, _u16p), _p(s, _f32p), R, K, _p(Xq, _i8p), _p(sX, _f32p))
    return Xq, sX[:R]


def sq_linear(X, s, Wq, sW, stages: bool = False):
    """Y fp16 [R,N] of the smoothed W8A8 product (no outlier decomposition)."""
    Xq, sX = sq_quantize_rows(X, s)
    acc = int8_gemm(Xq, Wq)
    R, N = acc.shape
    Y = np.empty((R, N), np.uint16)
    sW = np.ascontiguousarray(sW, dtype=np.float32)
    lib().oracle_sq_output(_p(acc, _i32p), _p(np.ascontiguousarray(sX, np.float32), _f32p),
                           _p(sW, _f32p), R, N, _p(Y, _u16p))
    Y = Y.view(np.float16)
    if not stages:
        return Y
    return dict(Y=Y, Xq=Xq, sX=sX, acc=acc)
