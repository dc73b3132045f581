"""LLM.int8() mixed-precision linear layer for AMD Instinct MI355X (gfx950).

A thin ctypes binding of ``libllm_int8.so`` (HIP kernels + C ABI, declared
in ``include/llm_int8.h``).  This module only marshals arguments: every step
of the computation runs in the library's kernels.  PyTorch provides the
device memory and the stream; calls are enqueued on torch's current stream
of the tensors' device and never synchronize.

    Wq, sW = quantize_weight(W)            # once per weight, W fp16 [N,K]
    Y = linear(X, Wq, sW, threshold=6.0)   # X fp16 [T,K] -> Y fp16 [T,N]

The method (hncyxsy.com/news/230290 "LLM quantization, part 2", section
2.1; lowentro.cn "model quantization" notes, Q4; tqpw.cn/news/5683,
sections 2.1 and 3.1): feature columns of X with some |x| > threshold are
outliers and are multiplied in floating point; the other columns are
quantized to int8 with a per-token absmax scale (the weight with a
per-output-feature scale), multiplied as int8 x int8 -> int32, dequantized,
and added to the outlier product; the result is fp16.

If the library has not been built, every call raises; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "Int8MatmulError", "LibraryNotBuilt", "library_path", "load_library",
    "quantize_weight", "workspace_bytes", "linear_workspace_bytes", "plan", "new_workspace",
    "linear", "linear_noalloc", "NOALLOC_SCRATCH_BYTES", "prepare",
    "gemm", "export_stages", "stages", "few_token_path", "linear_fp16w", "prepare_fp16w",
    "gemm_fp16w", "smoothquant_column_absmax", "smoothquant_factors",
    "smoothquant_quantize_weight", "smoothquant_prepare", "smoothquant_linear",
    "cache_bytes", "new_cache", "cache_reset", "cache_stats", "linear_cached", "prepare_cached",
    "gemm_cached", "STATUS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libllm_int8.so")
_lib = None

STATUS = {
    0: "LI8_OK",
    1: "LI8_ERR_INVALID_ARG",
    2: "LI8_ERR_SHAPE",
    3: "LI8_ERR_ALIGN",
    4: "LI8_ERR_WORKSPACE",
    5: "LI8_ERR_HIP",
    6: "LI8_ERR_SCRATCH",
}


class Int8MatmulError(RuntimeError):
    """A library call returned a status other than LI8_OK."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")


class LibraryNotBuilt(ImportError):
    pass


def library_path() -> str:
    return _LIB_PATH


def load_library() -> ctypes.CDLL:
    """Load libllm_int8.so (raises LibraryNotBuilt if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise LibraryNotBuilt(
            f"{_LIB_PATH} is missing; build it with `python -m int8_matmul_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    L.li8_status_str.restype = ctypes.c_char_p
    L.li8_status_str.argtypes = [ctypes.c_int]
    L.int8_quantize_weight.restype = ctypes.c_int
    L.int8_quantize_weight.argtypes = [vp, i64, i64, vp, vp, vp]
    L.llm_int8_workspace_bytes.restype = sz
    L.llm_int8_workspace_bytes.argtypes = [i64, i64, i64]
    L.llm_int8_linear_workspace_bytes.restype = sz
    L.llm_int8_linear_workspace_bytes.argtypes = [i64, i64, i64]
    L.llm_int8_plan.restype = ctypes.c_int
    L.llm_int8_plan.argtypes = [i64, i64, i64, vp, vp, vp, vp, vp]
    L.llm_int8_linear.restype = ctypes.c_int
    L.llm_int8_linear.argtypes = [vp, vp, vp, ctypes.c_float, i64, i64, i64, vp, vp, sz, vp]
    L.llm_int8_linear_noalloc.restype = ctypes.c_int
    L.llm_int8_linear_noalloc.argtypes = [vp, vp, vp, ctypes.c_float, i64, i64, i64, vp, vp]
    L.llm_int8_prepare.restype = ctypes.c_int
    L.llm_int8_prepare.argtypes = [vp, vp, ctypes.c_float, i64, i64, i64, vp, sz, vp]
    L.llm_int8_gemm.restype = ctypes.c_int
    L.llm_int8_gemm.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, sz, vp]
    L.llm_int8_linear_fp16w.restype = ctypes.c_int
    L.llm_int8_linear_fp16w.argtypes = [vp, vp, vp, vp, ctypes.c_float, i64, i64, i64, vp, vp,
                                        sz, vp]
    L.llm_int8_prepare_fp16w.restype = ctypes.c_int
    L.llm_int8_prepare_fp16w.argtypes = [vp, vp, ctypes.c_float, i64, i64, i64, vp, sz, vp]
    L.llm_int8_gemm_fp16w.restype = ctypes.c_int
    L.llm_int8_gemm_fp16w.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, vp, sz, vp]
    L.smoothquant_column_absmax.restype = ctypes.c_int
    L.smoothquant_column_absmax.argtypes = [vp, i64, i64, vp, vp]
    L.smoothquant_factors.restype = ctypes.c_int
    L.smoothquant_factors.argtypes = [vp, vp, ctypes.c_double, i64, vp, vp, vp]
    L.smoothquant_quantize_weight.restype = ctypes.c_int
    L.smoothquant_quantize_weight.argtypes = [vp, vp, i64, i64, vp, vp, vp]
    L.smoothquant_prepare.restype = ctypes.c_int
    L.smoothquant_prepare.argtypes = [vp, vp, i64, i64, i64, vp, sz, vp]
    L.smoothquant_linear.restype = ctypes.c_int
    L.smoothquant_linear.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp, sz, vp]
    L.llm_int8_cache_bytes.restype = sz
    L.llm_int8_cache_bytes.argtypes = [i64, i64]
    L.llm_int8_cache_reset.restype = ctypes.c_int
    L.llm_int8_cache_reset.argtypes = [vp, sz, i64, i64, vp]
    L.llm_int8_linear_cached.restype = ctypes.c_int
    L.llm_int8_linear_cached.argtypes = [vp, vp, vp, ctypes.c_float, i64, i64, i64, vp, vp, sz,
                                         vp, sz, vp]
    L.llm_int8_prepare_cached.restype = ctypes.c_int
    L.llm_int8_prepare_cached.argtypes = [vp, vp, ctypes.c_float, i64, i64, i64, vp, sz, vp, sz,
                                          vp]
    L.llm_int8_gemm_cached.restype = ctypes.c_int
    L.llm_int8_gemm_cached.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp, sz, vp, sz, vp]
    L.llm_int8_export_stages.restype = ctypes.c_int
    L.llm_int8_export_stages.argtypes = [vp, sz, i64, i64, i64, vp, vp, vp, vp, vp, vp, vp]
    L.llm_int8_stages.restype = ctypes.c_int
    L.llm_int8_stages.argtypes = [vp, vp, vp, ctypes.c_float, i64, i64, i64, vp, vp, sz, vp, vp, vp,
                                  vp, vp, vp, vp, vp]
    _lib = L
    return L


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise Int8MatmulError(fn, status)


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _require(t: torch.Tensor, dtype: torch.dtype, name: str, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def quantize_weight(W: torch.Tensor, Wq: torch.Tensor | None = None,
                    sW: torch.Tensor | None = None):
    """Vector-wise int8 quantization of W fp16 [N,K]: (Wq int8 [N,K], sW fp32 [N])."""
    L = load_library()
    _require(W, torch.float16, "W", 2)
    N, K = W.shape
    if Wq is None:
        Wq = torch.empty((N, K), dtype=torch.int8, device=W.device)
    if sW is None:
        sW = torch.empty((N,), dtype=torch.float32, device=W.device)
    _check("int8_quantize_weight",
           L.int8_quantize_weight(_ptr(W), N, K, _ptr(Wq), _ptr(sW), _stream(W.device)))
    return Wq, sW


def workspace_bytes(T: int, K: int, N: int) -> int:
    n = load_library().llm_int8_workspace_bytes(T, K, N)
    if n == 0:
        raise Int8MatmulError("llm_int8_workspace_bytes", 2)
    return int(n)


def new_workspace(T: int, K: int, N: int, device) -> torch.Tensor:
    return torch.empty(workspace_bytes(T, K, N), dtype=torch.uint8, device=device)


def linear_workspace_bytes(T: int, K: int, N: int) -> int:
    """Bytes llm_int8_linear needs for this shape (0 on the few-token path)."""
    return int(load_library().llm_int8_linear_workspace_bytes(T, K, N))


PATHS = {0: "empty", 1: "few_tokens", 2: "tiled", 3: "few_tokens_split"}


def plan(T: int, K: int, N: int) -> dict:
    """Which kernels a call of this shape runs: path, output tile, and the
    outlier counts (fold_lo, fold_hi] for which the tiled GEMM copies the
    weight's outlier columns itself instead of the prepare kernel."""
    out = [ctypes.c_int32() for _ in range(5)]
    _check("llm_int8_plan", load_library().llm_int8_plan(T, K, N, *(ctypes.byref(o) for o in out)))
    path, tm, tn, lo, hi = (o.value for o in out)
    return dict(path=PATHS[path], tile_m=tm, tile_n=tn, fold_lo=lo, fold_hi=hi)


def few_token_path(T: int, K: int) -> bool:
    """True if ``linear`` runs on a few-token path (fused or split) for T x K."""
    return plan(T, K, 1)["path"] in ("few_tokens", "few_tokens_split")


def _ws(workspace, T, K, N, device):
    if workspace is None:
        workspace = new_workspace(T, K, N, device)
    _require(workspace, torch.uint8, "workspace", 1)
    return workspace


def linear(X: torch.Tensor, Wq: torch.Tensor, sW: torch.Tensor, threshold: float = 6.0,
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None):
    """Y fp16 [T,N] = the LLM.int8() decomposed product of X fp16 [T,K] and W."""
    L = load_library()
    _require(X, torch.float16, "X", 2)
    _require(Wq, torch.int8, "Wq", 2)
    _require(sW, torch.float32, "sW", 1)
    T, K = X.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K or sW.shape[0] != N:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, Wq {tuple(Wq.shape)}, sW {tuple(sW.shape)}")
    if out is None:
        out = torch.empty((T, N), dtype=torch.float16, device=X.device)
    _require(out, torch.float16, "out", 2)
    if workspace is None and linear_workspace_bytes(T, K, N) == 0:
        ws = torch.empty(0, dtype=torch.uint8, device=X.device)   # the fused path uses none
    else:
        ws = _ws(workspace, T, K, N, X.device)
    _check("llm_int8_linear",
           L.llm_int8_linear(_ptr(X), _ptr(Wq), _ptr(sW), float(threshold), T, K, N,
                             _ptr(out), _ptr(ws), ws.numel(), _stream(X.device)))
    return out


# Bytes of the fixed per-GPU array llm_int8_linear_noalloc works in.
NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024


def linear_noalloc(X: torch.Tensor, Wq: torch.Tensor, sW: torch.Tensor, threshold: float = 6.0,
                   out: torch.Tensor | None = None):
    """As ``linear``, with the library's fixed per-GPU scratch array as the
    workspace (llm_int8_linear_noalloc): the library allocates nothing.
    Pass ``out`` to allocate nothing here either."""
    L = load_library()
    _require(X, torch.float16, "X", 2)
    _require(Wq, torch.int8, "Wq", 2)
    _require(sW, torch.float32, "sW", 1)
    T, K = X.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K or sW.shape[0] != N:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, Wq {tuple(Wq.shape)}, sW {tuple(sW.shape)}")
    if out is None:
        out = torch.empty((T, N), dtype=torch.float16, device=X.device)
    _require(out, torch.float16, "out", 2)
    _check("llm_int8_linear_noalloc",
           L.llm_int8_linear_noalloc(_ptr(X), _ptr(Wq), _ptr(sW), float(threshold), T, K, N,
                                     _ptr(out), _stream(X.device)))
    return out


def prepare(X: torch.Tensor, Wq: torch.Tensor, threshold: float, workspace: torch.Tensor):
    """Detection, token quantization and outlier gathers into `workspace`."""
    L = load_library()
    _require(X, torch.float16, "X", 2)
    _require(Wq, torch.int8, "Wq", 2)
    T, K = X.shape
    N = Wq.shape[0]
    ws = _ws(workspace, T, K, N, X.device)
    _check("llm_int8_prepare",
           L.llm_int8_prepare(_ptr(X), _ptr(Wq), float(threshold), T, K, N, _ptr(ws),
                              ws.numel(), _stream(X.device)))
    return ws


def gemm(Wq: torch.Tensor, sW: torch.Tensor, T: int, workspace: torch.Tensor,
         out: torch.Tensor | None = None, acc: torch.Tensor | None = None):
    """int8 GEMM + epilogue reading what `prepare` left in `workspace`."""
    L = load_library()
    _require(Wq, torch.int8, "Wq", 2)
    _require(sW, torch.float32, "sW", 1)
    N, K = Wq.shape
    if out is None:
        out = torch.empty((T, N), dtype=torch.float16, device=Wq.device)
    _require(out, torch.float16, "out", 2)
    if acc is not None:
        _require(acc, torch.int32, "acc", 2)
    _require(workspace, torch.uint8, "workspace", 1)
    _check("llm_int8_gemm",
           L.llm_int8_gemm(_ptr(Wq), _ptr(sW), T, K, N, _ptr(out), _ptr(acc), _ptr(workspace),
                           workspace.numel(), _stream(Wq.device)))
    return out


def linear_fp16w(X: torch.Tensor, Wq: torch.Tensor, sW: torch.Tensor, W: torch.Tensor,
                 threshold: float = 6.0, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None):
    """The fp16-weight variant: the outlier columns multiply the fp16 weight
    W [N,K] (the one Wq, sW were quantized from) instead of Wq*sW."""
    L = load_library()
    _require(X, torch.float16, "X", 2)
    _require(Wq, torch.int8, "Wq", 2)
    _require(sW, torch.float32, "sW", 1)
    _require(W, torch.float16, "W", 2)
    T, K = X.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K or sW.shape[0] != N or tuple(W.shape) != (N, K):
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, Wq {tuple(Wq.shape)}, "
                         f"sW {tuple(sW.shape)}, W {tuple(W.shape)}")
    if out is None:
        out = torch.empty((T, N), dtype=torch.float16, device=X.device)
    _require(out, torch.float16, "out", 2)
    ws = _ws(workspace, T, K, N, X.device)
    _check("llm_int8_linear_fp16w",
           L.llm_int8_linear_fp16w(_ptr(X), _ptr(Wq), _ptr(sW), _ptr(W), float(threshold), T, K,
                                   N, _ptr(out), _ptr(ws), ws.numel(), _stream(X.device)))
    return out


def prepare_fp16w(X: torch.Tensor, W: torch.Tensor, threshold: float, workspace: torch.Tensor):
    """`prepare` of the fp16-weight variant (gathers the outlier columns of W)."""
    L = load_library()
    _require(X, torch.float16, "X", 2)
    _require(W, torch.float16, "W", 2)
    T, K = X.shape
    N = W.shape[0]
    ws = _ws(workspace, T, K, N, X.device)
    _check("llm_int8_prepare_fp16w",
           L.llm_int8_prepare_fp16w(_ptr(X), _ptr(W), float(threshold), T, K, N, _ptr(ws),
                                    ws.numel(), _stream(X.device)))
    return ws


def gemm_fp16w(Wq: torch.Tensor, sW: torch.Tensor, W: torch.Tensor, T: int,
               workspace: torch.Tensor, out: torch.Tensor | None = None,
               acc: torch.Tensor | None = None):
    """`gemm` of the fp16-weight variant, on a workspace from `prepare_fp16w`."""
    L = load_library()
    _require(Wq, torch.int8, "Wq", 2)
    _require(sW, torch.float32, "sW", 1)
    _require(W, torch.float16, "W", 2)
    N, K = Wq.shape
    if out is None:
        out = torch.empty((T, N), dtype=torch.float16, device=Wq.device)
    _require(out, torch.float16, "out", 2)
    if acc is not None:
        _require(acc, torch.int32, "acc", 2)
    _require(workspace, torch.uint8, "workspace", 1)
    _check("llm_int8_gemm_fp16w",
           L.llm_int8_gemm_fp16w(_ptr(Wq), _ptr(sW), _ptr(W), T, K, N, _ptr(out), _ptr(acc),
                                 _ptr(workspace), workspace.numel(), _stream(Wq.device)))
    return out


def cache_bytes(K: int, N: int) -> int:
    n = load_library().llm_int8_cache_bytes(K, N)
    if n == 0:
        raise Int8MatmulError("llm_int8_cache_bytes", 2)
    return int(n)


def new_cache(K: int, N: int, device) -> torch.Tensor:
    """An empty outlier-column cache for a weight [N,K] (reset, ready to use)."""
    c = torch.empty(cache_bytes(K, N), dtype=torch.uint8, device=device)
    cache_reset(c, K, N)
    return c


def cache_reset(cache: torch.Tensor, K: int, N: int) -> torch.Tensor:
    """Mark the cache empty; needed after its weight changes."""
    L = load_library()
    _require(cache, torch.uint8, "cache", 1)
    _check("llm_int8_cache_reset",
           L.llm_int8_cache_reset(_ptr(cache), cache.numel(), K, N, _stream(cache.device)))
    return cache


def cache_stats(cache: torch.Tensor) -> dict:
    """valid, nO, hits, misses from the cache header (synchronizes)."""
    h = cache[:16].view(torch.int32).cpu().tolist()
    return dict(valid=h[0], nO=h[1], hits=h[2], misses=h[3])


def linear_cached(X: torch.Tensor, Wq: torch.Tensor, sW: torch.Tensor, cache: torch.Tensor,
                  threshold: float = 6.0, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None):
    """`linear` with an outlier-column cache bound to Wq (bit-identical Y)."""
    L = load_library()
    _require(X, torch.float16, "X", 2)
    _require(Wq, torch.int8, "Wq", 2)
    _require(sW, torch.float32, "sW", 1)
    _require(cache, torch.uint8, "cache", 1)
    T, K = X.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K or sW.shape[0] != N:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, Wq {tuple(Wq.shape)}, sW {tuple(sW.shape)}")
    if out is None:
        out = torch.empty((T, N), dtype=torch.float16, device=X.device)
    _require(out, torch.float16, "out", 2)
    ws = _ws(workspace, T, K, N, X.device)
    _check("llm_int8_linear_cached",
           L.llm_int8_linear_cached(_ptr(X), _ptr(Wq), _ptr(sW), float(threshold), T, K, N,
                                    _ptr(out), _ptr(ws), ws.numel(), _ptr(cache), cache.numel(),
                                    _stream(X.device)))
    return out


def prepare_cached(X: torch.Tensor, Wq: torch.Tensor, threshold: float, workspace: torch.Tensor,
                   cache: torch.Tensor):
    """`prepare` with an outlier-column cache."""
    L = load_library()
    _require(X, torch.float16, "X", 2)
    _require(Wq, torch.int8, "Wq", 2)
    _require(cache, torch.uint8, "cache", 1)
    T, K = X.shape
    N = Wq.shape[0]
    ws = _ws(workspace, T, K, N, X.device)
    _check("llm_int8_prepare_cached",
           L.llm_int8_prepare_cached(_ptr(X), _ptr(Wq), float(threshold), T, K, N, _ptr(ws),
                                     ws.numel(), _ptr(cache), cache.numel(), _stream(X.device)))
    return ws


def gemm_cached(Wq: torch.Tensor, sW: torch.Tensor, T: int, workspace: torch.Tensor,
                cache: torch.Tensor, out: torch.Tensor | None = None,
                acc: torch.Tensor | None = None):
    """`gemm` on a workspace from `prepare_cached` with the same cache."""
    L = load_library()
    _require(Wq, torch.int8, "Wq", 2)
    _require(sW, torch.float32, "sW", 1)
    _require(cache, torch.uint8, "cache", 1)
    N, K = Wq.shape
    if out is None:
        out = torch.empty((T, N), dtype=torch.float16, device=Wq.device)
    _require(out, torch.float16, "out", 2)
    if acc is not None:
        _require(acc, torch.int32, "acc", 2)
    _require(workspace, torch.uint8, "workspace", 1)
    _check("llm_int8_gemm_cached",
           L.llm_int8_gemm_cached(_ptr(Wq), _ptr(sW), T, K, N, _ptr(out), _ptr(acc),
                                  _ptr(workspace), workspace.numel(), _ptr(cache), cache.numel(),
                                  _stream(Wq.device)))
    return out


def smoothquant_column_absmax(A: torch.Tensor, out: torch.Tensor | None = None):
    """max_r |A[r,j]| per column of fp16 A [rows,K], as fp32 [K]."""
    L = load_library()
    _require(A, torch.float16, "A", 2)
    rows, K = A.shape
    if out is None:
        out = torch.empty((K,), dtype=torch.float32, device=A.device)
    _require(out, torch.float32, "out", 1)
    _check("smoothquant_column_absmax",
           L.smoothquant_column_absmax(_ptr(A), rows, K, _ptr(out), _stream(A.device)))
    return out


def smoothquant_factors(ax: torch.Tensor, aw: torch.Tensor, alpha: float = 0.5):
    """(s, s_inv) fp32 [K]: s_j = ax_j^alpha / aw_j^(1-alpha) (1 where either
    maximum is 0) and fl32(1/s_j)."""
    L = load_library()
    _require(ax, torch.float32, "ax", 1)
    _require(aw, torch.float32, "aw", 1)
    K = ax.shape[0]
    if aw.shape[0] != K:
        raise ValueError(f"shape mismatch: ax {tuple(ax.shape)}, aw {tuple(aw.shape)}")
    s = torch.empty((K,), dtype=torch.float32, device=ax.device)
    s_inv = torch.empty((K,), dtype=torch.float32, device=ax.device)
    _check("smoothquant_factors",
           L.smoothquant_factors(_ptr(ax), _ptr(aw), float(alpha), K, _ptr(s), _ptr(s_inv),
                                 _stream(ax.device)))
    return s, s_inv


def smoothquant_quantize_weight(W: torch.Tensor, s: torch.Tensor):
    """(Wq int8 [N,K], sW fp32 [N]) of the smoothed weight fl32(W * s)."""
    L = load_library()
    _require(W, torch.float16, "W", 2)
    _require(s, torch.float32, "s", 1)
    N, K = W.shape
    if s.shape[0] != K:
        raise ValueError(f"shape mismatch: W {tuple(W.shape)}, s {tuple(s.shape)}")
    Wq = torch.empty((N, K), dtype=torch.int8, device=W.device)
    sW = torch.empty((N,), dtype=torch.float32, device=W.device)
    _check("smoothquant_quantize_weight",
           L.smoothquant_quantize_weight(_ptr(W), _ptr(s), N, K, _ptr(Wq), _ptr(sW),
                                         _stream(W.device)))
    return Wq, sW


def smoothquant_prepare(X: torch.Tensor, s_inv: torch.Tensor, N: int, workspace: torch.Tensor):
    """Smoothed token codes and scales of X into `workspace` (no outlier
    column); `gemm` on it then gives the smoothed W8A8 product."""
    L = load_library()
    _require(X, torch.float16, "X", 2)
    _require(s_inv, torch.float32, "s_inv", 1)
    T, K = X.shape
    if s_inv.shape[0] != K:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, s_inv {tuple(s_inv.shape)}")
    ws = _ws(workspace, T, K, N, X.device)
    _check("smoothquant_prepare",
           L.smoothquant_prepare(_ptr(X), _ptr(s_inv), T, K, N, _ptr(ws), ws.numel(),
                                 _stream(X.device)))
    return ws


def smoothquant_linear(X: torch.Tensor, s_inv: torch.Tensor, Wq: torch.Tensor,
                       sW: torch.Tensor, out: torch.Tensor | None = None,
                       workspace: torch.Tensor | None = None):
    """Y fp16 [T,N] of the smoothed W8A8 product (SmoothQuant-style)."""
    L = load_library()
    _require(X, torch.float16, "X", 2)
    _require(s_inv, torch.float32, "s_inv", 1)
    _require(Wq, torch.int8, "Wq", 2)
    _require(sW, torch.float32, "sW", 1)
    T, K = X.shape
    N = Wq.shape[0]
    if Wq.shape[1] != K or sW.shape[0] != N or s_inv.shape[0] != K:
        raise ValueError(f"shape mismatch: X {tuple(X.shape)}, s_inv {tuple(s_inv.shape)}, "
                         f"Wq {tuple(Wq.shape)}, sW {tuple(sW.shape)}")
    if out is None:
        out = torch.empty((T, N), dtype=torch.float16, device=X.device)
    _require(out, torch.float16, "out", 2)
    ws = _ws(workspace, T, K, N, X.device)
    _check("smoothquant_linear",
           L.smoothquant_linear(_ptr(X), _ptr(s_inv), _ptr(Wq), _ptr(sW), T, K, N, _ptr(out),
                                _ptr(ws), ws.numel(), _stream(X.device)))
    return out


def export_stages(workspace: torch.Tensor, T: int, K: int, N: int) -> dict:
    """Device copies of the intermediate results of the last `prepare`."""
    L = load_library()
    _require(workspace, torch.uint8, "workspace", 1)
    dev = workspace.device
    nw = max((K + 31) // 32, 1)
    r = dict(
        outlier_bits=torch.empty(nw, dtype=torch.int32, device=dev),
        n_outliers=torch.empty(1, dtype=torch.int32, device=dev),
        outlier_idx=torch.empty(max(K, 1), dtype=torch.int32, device=dev),
        Xq=torch.empty((T, K), dtype=torch.int8, device=dev),
        sX=torch.empty(max(T, 1), dtype=torch.float32, device=dev),
        # gathered outlier values in 16-column chunks (see llm_int8.h)
        X_out=torch.empty(max(T * K, 1), dtype=torch.float16, device=dev),
    )
    _check("llm_int8_export_stages",
           L.llm_int8_export_stages(_ptr(workspace), workspace.numel(), T, K, N,
                                    _ptr(r["outlier_bits"]), _ptr(r["n_outliers"]),
                                    _ptr(r["outlier_idx"]), _ptr(r["Xq"]), _ptr(r["sX"]),
                                    _ptr(r["X_out"]), _stream(dev)))
    return r


def stages(X: torch.Tensor, Wq: torch.Tensor, sW: torch.Tensor, threshold: float,
           workspace: torch.Tensor | None = None) -> dict:
    """Y and every intermediate result of one call (llm_int8_stages)."""
    L = load_library()
    _require(X, torch.float16, "X", 2)
    _require(Wq, torch.int8, "Wq", 2)
    _require(sW, torch.float32, "sW", 1)
    T, K = X.shape
    N = Wq.shape[0]
    dev = X.device
    ws = _ws(workspace, T, K, N, dev)
    r = dict(
        Y=torch.empty((T, N), dtype=torch.float16, device=dev),
        flags=torch.empty(max(K, 1), dtype=torch.uint8, device=dev),
        n_outliers=torch.empty(1, dtype=torch.int32, device=dev),
        outlier_idx=torch.empty(max(K, 1), dtype=torch.int32, device=dev),
        Xq=torch.empty((T, K), dtype=torch.int8, device=dev),
        sX=torch.empty(max(T, 1), dtype=torch.float32, device=dev),
        X_out=torch.empty((T, K), dtype=torch.float16, device=dev),
        acc=torch.empty((T, N), dtype=torch.int32, device=dev),
    )
    _check("llm_int8_stages",
           L.llm_int8_stages(_ptr(X), _ptr(Wq), _ptr(sW), float(threshold), T, K, N, _ptr(r["Y"]),
                             _ptr(ws), ws.numel(), _ptr(r["flags"]), _ptr(r["n_outliers"]),
                             _ptr(r["outlier_idx"]), _ptr(r["Xq"]), _ptr(r["sX"]),
                             _ptr(r["X_out"]), _ptr(r["acc"]), _stream(dev)))
    return r
