"""The C ABI library: it loads, exports every declared symbol, and rejects bad
arguments on the host with the documented status before launching anything.

These run without a GPU: every call here fails validation, and validation
makes no HIP call.
"""
import ctypes
import math
import os
import re

import pytest

import int8_matmul_amd as li8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llm_int8.h")

OK, INVALID, SHAPE, ALIGN, WORKSPACE, SCRATCH = 0, 1, 2, 3, 4, 6
# fake, never-dereferenced device addresses
P = 0x7F0000000000
P2 = 0x7F0000100000
MIS = 0x7F0000000008  # 8-byte aligned only


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z][a-z0-9_]*)\s*\(", src)) - {"defined"})


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(li8.library_path()):
        import int8_matmul_amd.build as b
        b.build()
    return li8.load_library()


def test_header_declares_the_expected_entry_points():
    assert declared_functions() == sorted([
        "li8_status_str", "int8_quantize_weight", "llm_int8_workspace_bytes",
        "llm_int8_linear_workspace_bytes", "llm_int8_plan", "llm_int8_linear_noalloc",
        "llm_int8_linear", "llm_int8_prepare", "llm_int8_gemm", "llm_int8_export_stages",
        "llm_int8_stages",
        "llm_int8_linear_fp16w", "llm_int8_prepare_fp16w", "llm_int8_gemm_fp16w",
        "smoothquant_column_absmax", "smoothquant_factors", "smoothquant_quantize_weight",
        "smoothquant_prepare", "smoothquant_linear",
        "llm_int8_cache_bytes", "llm_int8_cache_reset", "llm_int8_linear_cached",
        "llm_int8_prepare_cached", "llm_int8_gemm_cached",
    ])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    # and they are C symbols (no C++ mangling)
    raw = ctypes.CDLL(li8.library_path())
    for name in declared_functions():
        ctypes.cast(getattr(raw, name), ctypes.c_void_p)


def test_status_strings(lib):
    for code, name in li8.STATUS.items():
        assert lib.li8_status_str(code).decode() == name
    assert lib.li8_status_str(99).decode() == "LI8_UNKNOWN_STATUS"


def test_workspace_bytes(lib):
    ws = lib.llm_int8_workspace_bytes
    assert ws(16, 17, 16) == 0          # K % 16
    assert ws(-1, 16, 16) == 0
    assert ws(16, 133152, 16) == 0      # K above the int32 bound
    assert ws(16, 133136, 16) > 0
    a = ws(4096, 4096, 11008)
    # covers Xq (T*K), the gathered outlier columns of X (2*T*K) and of the
    # weight (2*N*K: fp16 in the fp16-weight variant) in the worst case
    # nO = K, plus small tables
    assert a >= 4096 * 4096 * 3 + 2 * 11008 * 4096
    assert a < 4096 * 4096 * 3 + 2 * 11008 * 4096 + (1 << 20)
    assert ws(0, 16, 16) > 0 and ws(16, 0, 16) > 0
    assert ws(8, 4096, 4096) <= ws(16, 4096, 4096) <= ws(16, 4096, 8192)
    assert a % 256 == 0


def test_linear_workspace_bytes(lib):
    """llm_int8_linear needs no workspace on the few-token path, and the
    int8 layout (no fp16 weight columns) on the tiled path."""
    lw, ws = lib.llm_int8_linear_workspace_bytes, lib.llm_int8_workspace_bytes
    assert lw(8, 4096, 11008) == 0 and lw(16, 8192, 28672) == 0 and lw(1, 16, 1) == 0
    assert lw(0, 4096, 16) == 0 and lw(16, 17, 16) == 0
    a = lw(4096, 4096, 11008)
    assert 4096 * 4096 * 3 + 11008 * 4096 <= a < 4096 * 4096 * 3 + 11008 * 4096 + (1 << 20)
    assert ws(4096, 4096, 11008) - a >= 11008 * 4096
    assert lw(17, 4096, 64) > 0 and lw(8, 8208, 64) > 0   # past either few-token bound


def test_plan(lib):
    few = dict(fold_lo=0, fold_hi=0)
    assert li8.plan(8, 4096, 4096) == dict(path="few_tokens", tile_m=8, tile_n=16, **few)
    assert li8.plan(0, 4096, 4096)["path"] == "empty"
    p = li8.plan(4096, 4096, 11008)
    assert p["path"] == "tiled" and p["tile_m"] == 256 and p["tile_n"] in (128, 192, 256)
    # only 128-wide tiles copy the weight's outlier columns, for 64 < nO <= 256
    assert p["tile_n"] == 128 or (p["fold_lo"], p["fold_hi"]) == (0, 0)
    assert li8.plan(512, 5120, 13824) == dict(path="tiled", tile_m=256, tile_n=128,
                                              fold_lo=64, fold_hi=256)
    # not past K = 8192, where the bit set no longer fits the GEMM's LDS copy
    assert li8.plan(4096, 8208, 4096)["fold_hi"] == 0
    assert li8.plan(17, 16, 16)["path"] == "tiled"
    with pytest.raises(li8.Int8MatmulError):
        li8.plan(16, 24, 16)
    o = [ctypes.c_int32() for _ in range(5)]
    refs = [ctypes.byref(v) for v in o]
    for i in range(5):
        args = refs[:i] + [None] + refs[i + 1:]
        assert lib.llm_int8_plan(4, 16, 4, *args) == INVALID
    assert li8.few_token_path(16, 8192) and not li8.few_token_path(17, 8192)
    assert li8.plan(8, 11008, 4096) == dict(path="few_tokens_split", tile_m=8, tile_n=16, **few)
    assert li8.few_token_path(16, 8208) and li8.plan(16, 8208, 5)["path"] == "few_tokens_split"


def test_quantize_weight_validation(lib):
    f = lib.int8_quantize_weight
    assert f(P, 4, 17, P, P, None) == SHAPE
    assert f(P, -1, 16, P, P, None) == SHAPE
    assert f(None, 4, 16, P, P, None) == INVALID
    assert f(P, 4, 16, None, P, None) == INVALID
    assert f(P, 4, 16, P, None, None) == INVALID
    assert f(MIS, 4, 16, P, P, None) == ALIGN
    assert f(P, 4, 16, P, MIS, None) == ALIGN
    assert f(None, 0, 16, None, None, None) == OK   # empty: nothing to do


def test_linear_validation(lib):
    f = lib.llm_int8_linear
    need = lib.llm_int8_workspace_bytes(32, 64, 48)
    args = dict(X=P, Wq=P, sW=P, thr=6.0, T=32, K=64, N=48, Y=P2, ws=P, wsb=need)

    def call(**kw):
        a = dict(args, **kw)
        return f(a["X"], a["Wq"], a["sW"], a["thr"], a["T"], a["K"], a["N"], a["Y"],
                 a["ws"], a["wsb"], None)

    assert call(K=24) == SHAPE
    assert call(T=-3) == SHAPE
    assert call(K=133152) == SHAPE
    assert call(thr=-1.0) == INVALID
    assert call(thr=math.nan) == INVALID
    assert call(X=None) == INVALID
    assert call(Wq=None) == INVALID
    assert call(sW=None) == INVALID
    assert call(Y=None) == INVALID
    assert call(X=MIS) == ALIGN
    assert call(Y=MIS) == ALIGN
    assert call(ws=MIS) == ALIGN
    assert call(ws=None) == WORKSPACE
    # the int8 path does not need the fp16-weight variant's larger layout
    need8 = lib.llm_int8_linear_workspace_bytes(32, 64, 48)
    assert 0 < need8 < need
    assert call(wsb=need8 - 1) == WORKSPACE
    # few tokens: no workspace needed, but a misaligned one is still refused
    assert call(T=8, ws=MIS) == ALIGN
    assert call(T=8, X=None, ws=None, wsb=0) == INVALID
    # empty calls are valid and enqueue nothing, whatever the pointers
    assert call(T=0, X=None, Y=None, ws=None, wsb=0) == OK
    assert call(N=0, Wq=None, sW=None, Y=None, ws=None, wsb=0) == OK
    assert call(T=0, thr=math.inf) == OK
    assert call(T=0, thr=-0.0) == OK


def test_noalloc_validation(lib):
    """The allocation-free linear: argument checks as for llm_int8_linear,
    and shapes whose workspace exceeds the fixed array refused before
    anything is looked up or launched."""
    f = lib.llm_int8_linear_noalloc
    assert f(P, P, P, 6.0, 32, 24, 48, P2, None) == SHAPE
    assert f(None, P, P, 6.0, 32, 64, 48, P2, None) == INVALID
    assert f(P, P, P, math.nan, 32, 64, 48, P2, None) == INVALID
    assert f(P, P, MIS, 6.0, 32, 64, 48, P2, None) == ALIGN
    assert f(P, P, P, 6.0, 32, 64, 48, None, None) == INVALID
    assert f(None, None, None, 6.0, 0, 64, 48, None, None) == OK   # empty
    # 70B slice: about 336 MB of workspace against the 128 MiB array
    assert lib.llm_int8_linear_workspace_bytes(4096, 8192, 28672) > li8.NOALLOC_SCRATCH_BYTES
    assert f(P, P, P, 6.0, 4096, 8192, 28672, P2, None) == SCRATCH
    assert lib.llm_int8_linear_workspace_bytes(4096, 4096, 11008) <= li8.NOALLOC_SCRATCH_BYTES
    assert lib.li8_status_str(SCRATCH).decode() == "LI8_ERR_SCRATCH"


def test_prepare_and_gemm_validation(lib):
    need = lib.llm_int8_workspace_bytes(32, 64, 48)
    need8 = lib.llm_int8_linear_workspace_bytes(32, 64, 48)
    p = lib.llm_int8_prepare
    assert p(None, P, 6.0, 32, 64, 48, P, need, None) == INVALID
    assert p(P, P, math.nan, 32, 64, 48, P, need, None) == INVALID
    assert p(P, P, 6.0, 32, 64, 48, P, need8 - 1, None) == WORKSPACE
    assert p(P, P, 6.0, 32, 72, 48, P, need, None) == SHAPE
    g = lib.llm_int8_gemm
    assert g(P, P, 32, 64, 48, None, None, P, need, None) == INVALID
    assert g(P, P, 32, 64, 48, P2, MIS, P, need, None) == ALIGN
    assert g(P, P, 32, 64, 48, P2, None, P, 16, None) == WORKSPACE
    assert g(P, P, 32, 64, 48, P2, None, P, need8 - 1, None) == WORKSPACE
    assert g(P, P, 0, 64, 48, None, None, None, 0, None) == OK
    # the fp16-weight variant needs the wider layout
    assert lib.llm_int8_gemm_fp16w(P, P, P, 32, 64, 48, P2, None, P, need - 1, None) == WORKSPACE
    assert lib.llm_int8_prepare_fp16w(P, P, 6.0, 32, 64, 48, P, need - 1, None) == WORKSPACE
    e = lib.llm_int8_export_stages
    assert e(None, 0, 32, 64, 48, None, None, None, None, None, None, None) == WORKSPACE
    assert e(P, need, 32, 65, 48, None, None, None, None, None, None, None) == SHAPE
    # the whole-call stage export checks everything before enqueueing anything
    s = lib.llm_int8_stages
    outs = (P, P, P, P, P, P, P)   # flags, nO, idx, Xq, sX, X_out, acc
    assert s(None, P, P, 6.0, 32, 64, 48, P2, P, need, *outs, None) == INVALID
    assert s(P, P, None, 6.0, 32, 64, 48, P2, P, need, *outs, None) == INVALID
    assert s(P, P, P, math.nan, 32, 64, 48, P2, P, need, *outs, None) == INVALID
    assert s(P, P, P, 6.0, 32, 64, 48, None, P, need, *outs, None) == INVALID
    assert s(P, P, P, 6.0, 32, 72, 48, P2, P, need, *outs, None) == SHAPE
    assert s(P, P, P, 6.0, 32, 64, 48, P2, P, need8 - 1, *outs, None) == WORKSPACE
    assert s(P, P, P, 6.0, 32, 64, 48, P2, P, need, P, P, P, MIS, P, P, P, None) == ALIGN
    assert s(P, P, P, 6.0, 32, 64, 48, P2, P, need, P, P, P, P, P, MIS, P, None) == ALIGN
    assert s(P, P, P, 6.0, 32, 64, 48, P2, P, need, P, P, P, P, P, P, MIS, None) == ALIGN
    assert s(P, P, P, 6.0, 0, 64, 48, P2, P, need, *outs, None) == OK   # empty call


def test_fp16w_validation(lib):
    need = lib.llm_int8_workspace_bytes(32, 64, 48)
    f = lib.llm_int8_linear_fp16w
    assert f(P, P, P, None, 6.0, 32, 64, 48, P2, P, need, None) == INVALID   # no W
    assert f(P, P, P, MIS, 6.0, 32, 64, 48, P2, P, need, None) == ALIGN
    assert f(P, P, P, P, math.nan, 32, 64, 48, P2, P, need, None) == INVALID
    assert f(P, P, P, P, 6.0, 32, 72, 48, P2, P, need, None) == SHAPE
    assert f(None, None, None, None, 6.0, 0, 64, 48, None, None, 0, None) == OK
    g = lib.llm_int8_gemm_fp16w
    assert g(P, P, None, 32, 64, 48, P2, None, P, need, None) == INVALID
    assert g(P, P, MIS, 32, 64, 48, P2, None, P, need, None) == ALIGN
    p = lib.llm_int8_prepare_fp16w
    assert p(P, None, 6.0, 32, 64, 48, P, need, None) == INVALID
    assert p(P, MIS, 6.0, 32, 64, 48, P, need, None) == ALIGN


def test_smoothquant_validation(lib):
    c = lib.smoothquant_column_absmax
    assert c(P, 10, 72, P2, None) == SHAPE          # K % 16
    assert c(P, -1, 64, P2, None) == SHAPE
    assert c(P, 1 << 31, 64, P2, None) == SHAPE
    assert c(None, 10, 64, P2, None) == INVALID
    assert c(P, 10, 64, None, None) == INVALID
    assert c(MIS, 10, 64, P2, None) == ALIGN
    assert c(None, 10, 0, None, None) == OK         # K = 0: nothing to do
    f = lib.smoothquant_factors
    for bad in (-0.1, 1.5, math.nan):
        assert f(P, P, bad, 64, P2, P2, None) == INVALID
    assert f(P, None, 0.5, 64, P2, P2, None) == INVALID
    assert f(P, P, 0.5, 64, P2, None, None) == INVALID
    assert f(P, MIS, 0.5, 64, P2, P2, None) == ALIGN
    assert f(P, P, 0.5, 40, P2, P2, None) == SHAPE
    assert f(None, None, 0.5, 0, None, None, None) == OK
    q = lib.smoothquant_quantize_weight
    assert q(P, None, 48, 64, P2, P2, None) == INVALID
    assert q(P, P, 48, 64, P2, MIS, None) == ALIGN
    assert q(P, P, 48, 70, P2, P2, None) == SHAPE
    assert q(None, None, 0, 64, None, None, None) == OK
    need = lib.llm_int8_workspace_bytes(32, 64, 48)
    p = lib.smoothquant_prepare
    assert p(P, None, 32, 64, 48, P, need, None) == INVALID
    assert p(P, MIS, 32, 64, 48, P, need, None) == ALIGN
    assert p(P, P, 32, 64, 48, P, lib.llm_int8_linear_workspace_bytes(32, 64, 48) - 1,
             None) == WORKSPACE
    assert p(None, None, 0, 64, 48, None, 0, None) == OK
    L = lib.smoothquant_linear
    assert L(P, P, P, None, 32, 64, 48, P2, P, need, None) == INVALID   # no sW
    assert L(P, P, P, P, 32, 64, 48, None, P, need, None) == INVALID    # no Y
    assert L(P, P, P, P, 32, 64, 48, P2, None, need, None) == WORKSPACE
    assert L(P, P, MIS, P, 32, 64, 48, P2, P, need, None) == ALIGN
    assert L(P, P, P, P, 32, 65, 48, P2, P, need, None) == SHAPE
    assert L(None, None, None, None, 32, 64, 0, None, None, 0, None) == OK


def test_cache_validation(lib):
    assert lib.llm_int8_cache_bytes(72, 48) == 0            # K % 16
    cb = lib.llm_int8_cache_bytes(64, 48)
    assert cb >= 64 * 48 + 256
    r = lib.llm_int8_cache_reset
    assert r(None, cb, 64, 48, None) == INVALID
    assert r(MIS, cb, 64, 48, None) == ALIGN
    assert r(P, cb - 1, 64, 48, None) == WORKSPACE
    need = lib.llm_int8_workspace_bytes(32, 64, 48)
    L = lib.llm_int8_linear_cached
    assert L(P, P, P, 6.0, 32, 64, 48, P2, P, need, None, cb, None) == INVALID
    assert L(P, P, P, 6.0, 32, 64, 48, P2, P, need, MIS, cb, None) == ALIGN
    assert L(P, P, P, 6.0, 32, 64, 48, P2, P, need, P2, cb - 1, None) == WORKSPACE
    assert L(P, P, P, math.nan, 32, 64, 48, P2, P, need, P2, cb, None) == INVALID
    assert L(None, None, None, 6.0, 0, 64, 48, None, None, 0, None, 0, None) == OK
    p = lib.llm_int8_prepare_cached
    assert p(P, P, 6.0, 32, 64, 48, P, need, None, cb, None) == INVALID
    assert p(P, P, 6.0, 32, 64, 48, P, need, P2, 0, None) == WORKSPACE
    g = lib.llm_int8_gemm_cached
    assert g(P, P, 32, 64, 48, P2, None, P, need, None, cb, None) == INVALID
    assert g(P, P, 32, 64, 48, P2, None, P, need, MIS, cb, None) == ALIGN


def test_python_binding_rejects_cpu_tensors(lib):
    import torch
    W = torch.zeros(4, 16, dtype=torch.float16)
    with pytest.raises(ValueError):
        li8.quantize_weight(W)
