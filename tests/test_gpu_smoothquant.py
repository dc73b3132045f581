"""Parity of the SmoothQuant-style W8A8 path (smoothquant_*) with the CPU oracle.

lowentro.cn notes Q9-Q10 and hncyxsy.com/news/230290, section 5.1:
per-channel factors s_j move the activation's range into the weight, X . W^T = (X / s) . (W * s)^T, and both
sides are quantized with the absmax int8 scheme, with no outlier split.
Bar: bit-exact column maxima, factors, reciprocals, codes, scales and int32
accumulators; fp16 Y bit-exact too, since both sides compute
fp16(fl32(fl32(acc*sX)*sW)) from identical integers and scales.

Every stage is checked on its own inputs from the oracle (the GPU stages
take the oracle's factors), so a mismatch names the stage.
"""
import dataclasses

import numpy as np
import pytest
import torch

import int8_matmul_amd as li8
import oracle
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    li8.load_library()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint16) if a.dtype == np.float16 else a.view(np.uint32)


def draw(T, K, N, seed, Tcal=64, name="tiny"):
    """X [T,K], a calibration batch [Tcal,K] from the same distribution (same
    fixed outlier columns) and W [N,K]."""
    w = workloads.WORKLOADS[name]
    Xall, _ = workloads.make_activation(w, seed=seed, T=T + Tcal, K=K)
    W = workloads.make_weight(w, seed=seed, N=N, K=K)
    return Xall[:T], Xall[T:], W


def check_factors(ax, aw, alpha, label):
    s_o = oracle.sq_factors(ax, aw, alpha)
    s_g, r_g = li8.smoothquant_factors(dev(ax), dev(aw), alpha)
    s_g, r_g = host(s_g), host(r_g)
    assert np.array_equal(bits(s_g), bits(s_o)), f"{label}: factors"
    with np.errstate(divide="ignore"):
        r_o = np.float32(1.0) / s_o
    assert np.array_equal(bits(r_g), bits(r_o)), f"{label}: reciprocals"
    return s_o, r_o


def check_all(X, Xcal, W, alpha, label):
    T, K = X.shape
    N = W.shape[0]
    print(f"case sq {label}: T={T} K={K} N={N} alpha={alpha}", flush=True)
    # calibration statistics
    ax_o = oracle.column_absmax(Xcal)
    aw_o = oracle.column_absmax(W)
    ax_g = host(li8.smoothquant_column_absmax(dev(Xcal)))
    aw_g = host(li8.smoothquant_column_absmax(dev(W)))
    assert np.array_equal(bits(ax_g), bits(ax_o)), "activation column maxima"
    assert np.array_equal(bits(aw_g), bits(aw_o)), "weight column maxima"
    s_o, r_o = check_factors(ax_o, aw_o, alpha, label)
    # smoothed weight
    Wq_o, sW_o = oracle.sq_quantize_weight(W, s_o)
    Wq_g, sW_g = li8.smoothquant_quantize_weight(dev(W), dev(s_o))
    assert np.array_equal(host(Wq_g), Wq_o), "weight codes"
    assert np.array_equal(bits(host(sW_g)), bits(sW_o)), "weight scales"
    # per-call token side and GEMM
    o = oracle.sq_linear(X, s_o, Wq_o, sW_o, stages=True)
    Xd, rd = dev(X), dev(r_o)
    ws = li8.new_workspace(T, K, N, DEV)
    li8.smoothquant_prepare(Xd, rd, N, ws)
    st = li8.export_stages(ws, T, K, N)
    assert int(host(st["n_outliers"])[0]) == 0
    assert np.array_equal(host(st["Xq"]), o["Xq"]), "token codes"
    assert np.array_equal(bits(host(st["sX"])[:T]), bits(o["sX"])), "token scales"
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    Y2 = li8.gemm(Wq_g, sW_g, T, ws, acc=acc)
    Y = li8.smoothquant_linear(Xd, rd, Wq_g, sW_g)
    assert np.array_equal(host(acc), o["acc"]), "int32 accumulators"
    assert np.array_equal(bits(host(Y)), bits(o["Y"])), "Y"
    assert np.array_equal(bits(host(Y2)), bits(o["Y"])), "prepare + gemm"
    return o


@pytest.mark.parametrize("alpha", [0.0, 0.5, 0.8, 1.0])
def test_tiny(alpha):
    X, Xcal, W = draw(16, 256, 256, seed=3)
    check_all(X, Xcal, W, alpha, "tiny")


@pytest.mark.parametrize("T,K,N", [
    (300, 272, 520),     # tiled GEMM, ragged everywhere
    (513, 1024, 769),
    (1000, 2064, 300),   # K of 8 chunks per thread + a partial one
    (8, 4096, 300),      # few-token GEMM
    (1, 16, 1),
    (16, 8192, 130),
])
def test_shapes(T, K, N):
    X, Xcal, W = draw(T, K, N, seed=T * 7 + K + N)
    check_all(X, Xcal, W, 0.5, f"{T}x{K}x{N}")


def test_long_rows():
    """K beyond what k_sq_rows keeps in registers (8*256*4 = 8192): the
    second pass re-reads the row."""
    X, Xcal, W = draw(40, 12288, 96, seed=5)
    check_all(X, Xcal, W, 0.5, "long rows")


def test_degenerate_columns_and_rows():
    """Zero columns (factor 1 from either side), an all-zero token row
    (scale 0, codes 0) and an all-zero weight row."""
    X, Xcal, W = draw(64, 512, 96, seed=9)
    X[:, 5] = 0
    Xcal[:, 5] = 0           # ax = 0
    W[:, 7] = 0              # aw = 0
    X[10] = 0                # token row of zeros
    W[20] = 0                # weight row of zeros
    o = check_all(X, Xcal, W, 0.5, "degenerate")
    assert o["sX"][10] == 0 and not o["Xq"][10].any()


def test_factor_kernel_edge_values():
    """Factors over maxima spanning fp16's whole range and exact zeros."""
    rng = np.random.default_rng(2)
    K = 4096
    ax = np.exp2(rng.uniform(-24, 16, K)).astype(np.float32)
    aw = np.exp2(rng.uniform(-24, 16, K)).astype(np.float32)
    ax[:7] = 0
    aw[5:12] = 0
    for alpha in (0.0, 0.25, 0.5, 0.85, 1.0):
        check_factors(ax, aw, alpha, f"edge alpha={alpha}")


def test_column_absmax_many_rows():
    """More rows than the kernel's 1024 row groups: several rows per group."""
    w = workloads.WORKLOADS["ffn_13b"]
    A, _ = workloads.make_activation(w, seed=4, T=3000, K=1040)
    assert np.array_equal(bits(host(li8.smoothquant_column_absmax(dev(A)))),
                          bits(oracle.column_absmax(A)))


def test_smoothing_helps_on_outlier_activations():
    """With fixed outlier columns the smoothed product is closer to the exact
    X.W^T than the plain absmax W8A8 product (outlier threshold +inf)."""
    w = dataclasses.replace(workloads.WORKLOADS["prefill_7b_ffn_up"], T=256 + 128, N=512)
    Xall, _ = workloads.make_activation(w, seed=11)
    X, Xcal = Xall[:256], Xall[256:]
    W = workloads.make_weight(w, seed=11)
    Xd, Wd = dev(X), dev(W)
    s, r = li8.smoothquant_factors(li8.smoothquant_column_absmax(dev(Xcal)),
                                   li8.smoothquant_column_absmax(Wd), 0.5)
    Wq, sW = li8.smoothquant_quantize_weight(Wd, s)
    Ys = host(li8.smoothquant_linear(Xd, r, Wq, sW)).astype(np.float64)
    Wq0, sW0 = li8.quantize_weight(Wd)
    Y0 = host(li8.linear(Xd, Wq0, sW0, float("inf"))).astype(np.float64)
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    es, e0 = np.abs(Ys - ref).mean(), np.abs(Y0 - ref).mean()
    print(f"mean |err|: smoothed {es:.4g}, plain absmax {e0:.4g}", flush=True)
    assert es < 0.5 * e0
