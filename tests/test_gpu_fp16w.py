"""Parity of the fp16-weight variant (llm_int8_*_fp16w) with the CPU oracle.

The variant multiplies the outlier columns of X by the original fp16 weight
instead of the dequantized int8 codes (the extracted weight sub-matrix of
hncyxsy.com/news/230290, section 2.1).  Bar, as for the int8 path:
bit-exact outlier set, codes, scales and int32 accumulators; fp16 Y within
1e-2*(1+|y|) of the oracle, bit-exact when there is no outlier column (both
sides then compute fp16(fl32(fl32(acc*sX)*sW))).
"""
import numpy as np
import pytest
import torch

import int8_matmul_amd as li8
import oracle
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = 1e-2


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


def rel_err(y, ref):
    y = y.astype(np.float64)
    ref = ref.astype(np.float64)
    return float(np.max(np.abs(y - ref) / (1.0 + np.abs(ref)))) if y.size else 0.0


def run(X, W, thr):
    T, K = X.shape
    N = W.shape[0]
    Xd, Wd = dev(X), dev(W)
    Wq, sW = li8.quantize_weight(Wd)
    ws = li8.new_workspace(T, K, N, DEV)
    li8.prepare_fp16w(Xd, Wd, thr, ws)
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    Y2 = li8.gemm_fp16w(Wq, sW, Wd, T, ws, acc=acc)
    Y = li8.linear_fp16w(Xd, Wq, sW, Wd, thr)
    Yi = li8.linear(Xd, Wq, sW, thr)
    return dict(Y=host(Y), Y2=host(Y2), Yi=host(Yi), acc=host(acc), Wq=host(Wq), sW=host(sW))


def check(X, W, thr, label):
    print(f"case {label}: T={X.shape[0]} K={X.shape[1]} N={W.shape[0]} thr={thr}", flush=True)
    g = run(X, W, thr)
    o = oracle.linear(X, g["Wq"], g["sW"], thr, stages=True, W16=W)
    assert np.array_equal(g["Y"].view(np.uint16), g["Y2"].view(np.uint16)), \
        "prepare+gemm and the fused call differ"
    assert np.array_equal(g["acc"], o["acc"]), "int32 accumulators"
    e = rel_err(g["Y"], o["Y"])
    assert e <= TOL, f"{label}: fp16 output error {e}"
    if o["nO"] == 0:
        assert np.array_equal(g["Y"].view(np.uint16), o["Y"].view(np.uint16)), "no outliers: bit-exact"
        assert np.array_equal(g["Y"].view(np.uint16), g["Yi"].view(np.uint16)), "equals the int8 path"
    return g, o


@pytest.mark.parametrize("thr", [6.0, 0.0, np.inf])
def test_tiny(thr):
    X, W, _ = workloads.make("tiny")
    check(X, W, thr, f"tiny thr={thr}")


@pytest.mark.parametrize("T,K,N", [
    (300, 272, 520),     # tiled path, ragged everywhere
    (513, 1024, 769),
    (8, 4096, 300),      # few-token path
    (1, 16, 1),
    (16, 8192, 130),
    (8, 4096, 11008),    # several row groups per workgroup on the few-token path
    (8, 11008, 300),     # few tokens with K past the few-token kernel's bound
    (2050, 1040, 96),    # one wave per token row in the prepare kernel
])
@pytest.mark.parametrize("thr", [6.0, np.inf, 0.0])
def test_shapes(T, K, N, thr):
    w = workloads.WORKLOADS["tiny"]
    rng = np.random.default_rng(T * 13 + K * 7 + N)
    X, _ = workloads.make_activation(w, seed=int(rng.integers(1 << 30)), T=T, K=K)
    W = workloads.make_weight(w, seed=int(rng.integers(1 << 30)), N=N, K=K)
    check(X, W, thr, f"fp16w {T}x{K}x{N}")


def test_threshold_zero_is_the_fp16_product():
    """At threshold 0 the int8 part is empty: Y is X.W^T accumulated in fp32
    and rounded once to fp16."""
    rng = np.random.default_rng(21)
    X = rng.standard_normal((64, 256)).astype(np.float16)
    W = (rng.standard_normal((96, 256)) * 0.05).astype(np.float16)
    g, _ = check(X, W, 0.0, "threshold 0")
    ref = X.astype(np.float64) @ W.astype(np.float64).T
    assert rel_err(g["Y"], ref.astype(np.float16)) <= TOL


def test_many_outliers():
    w = workloads.WORKLOADS["ffn_13b"]
    import dataclasses
    w = dataclasses.replace(w, T=96, K=2048, N=384, sparse_rate=2e-3)
    X, _ = workloads.make_activation(w)
    W = workloads.make_weight(w)
    g, o = check(X, W, 6.0, "fp16w many outliers")
    assert o["nO"] > 200
