"""A seeded sweep of random shapes and thresholds through every entry point.

Each case draws T, K (a multiple of 16), N and the threshold from a fixed
seed, activations with fixed and token-sparse outlier columns, and checks
against the oracle:
  llm_int8_linear and prepare + gemm: bit-exact outlier set, codes, scales and
    int32 accumulators; Y within 1e-2*(1+|y|), bit-identical between the two
    routes, bit-exact against the oracle when there is no outlier column;
  llm_int8_linear_fp16w: accumulators bit-exact, Y within the tolerance;
  llm_int8_linear_cached: Y bit-identical to llm_int8_linear on a miss and
    on the following hit;
  smoothquant_linear: Y bit-exact against the oracle's smoothed product.
The shapes cover the tiled and the few-token paths and every output tile
shape of the GEMM (asserted), with ragged edges everywhere.
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
TOL = 1e-2
CASES = 48


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


def draw_shape(rng, i):
    """Every fourth case few tokens; every fourth (from 1) a wide layer of a
    few hundred to a thousand tokens and 4000-17000 features at small K, so
    that every output tile shape of the tiled GEMM is drawn; the rest small
    and ragged."""
    kind = i % 4
    if kind == 0:   # up to K = 19200, past the fused few-token kernel's 8192
        return int(rng.integers(1, 17)), 16 * int(rng.integers(1, 1201)), int(rng.integers(1, 900))
    if kind == 1:
        T, N = int(rng.integers(257, 1101)), int(rng.integers(4000, 17001))
        return T, 16 * int(rng.integers(1, 33)), N
    return int(rng.integers(17, 700)), 16 * int(rng.integers(1, 200)), int(rng.integers(1, 900))


def draw_case(i):
    rng = np.random.default_rng(1000 + i)
    T, K, N = draw_shape(rng, i)
    thr = float(rng.choice([6.0, 6.0, 3.0, 20.0, np.inf, 0.0]))
    w = dataclasses.replace(workloads.WORKLOADS["ffn_13b"], T=T, K=K, N=N,
                            n_fixed=int(min(K, rng.integers(0, 12))),
                            sparse_rate=float(rng.choice([0.0, 1e-4, 2e-3])))
    X, _ = workloads.make_activation(w, seed=int(rng.integers(1 << 30)))
    W = workloads.make_weight(w, seed=int(rng.integers(1 << 30)))
    return T, K, N, thr, X, W


def test_sweep_draws_every_path_and_tile():
    """The sweep's shapes reach both few-token paths and each tile shape of
    the tiled GEMM (as the library itself plans them)."""
    seen = set()
    for i in range(CASES):
        T, K, N = draw_shape(np.random.default_rng(1000 + i), i)
        p = li8.plan(T, K, N)
        seen.add((p["path"], p["tile_n"]))
    assert {("few_tokens", 16), ("few_tokens_split", 16), ("tiled", 128), ("tiled", 192),
            ("tiled", 256)} <= seen, seen


@pytest.mark.parametrize("i", range(CASES))
def test_sweep(i):
    T, K, N, thr, X, W = draw_case(i)
    print(f"case sweep {i}: T={T} K={K} N={N} thr={thr}", flush=True)
    Xd, Wd = dev(X), dev(W)
    Wq, sW = li8.quantize_weight(Wd)
    Wq_h, sW_h = host(Wq), host(sW)
    Wq_o, sW_o = oracle.quantize_weight(W)
    assert np.array_equal(Wq_h, Wq_o) and np.array_equal(sW_h.view(np.uint32), sW_o.view(np.uint32))

    # LLM.int8(): the whole call and its two halves
    o = oracle.linear(X, Wq_h, sW_h, thr, stages=True)
    Y = host(li8.linear(Xd, Wq, sW, thr))
    ws = li8.new_workspace(T, K, N, DEV)
    li8.prepare(Xd, Wq, thr, ws)
    st = li8.export_stages(ws, T, K, N)
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    Y2 = host(li8.gemm(Wq, sW, T, ws, acc=acc))
    nO = int(host(st["n_outliers"])[0])
    assert nO == o["nO"]
    assert np.array_equal(host(st["outlier_idx"])[:nO], o["idx"])
    assert np.array_equal(host(st["Xq"]), o["Xq"])
    assert np.array_equal(host(st["sX"])[:T].view(np.uint32), o["sX"].view(np.uint32))
    assert np.array_equal(host(acc), o["acc"])
    assert np.array_equal(Y.view(np.uint16), Y2.view(np.uint16)), "linear vs prepare + gemm"
    assert rel_err(Y, o["Y"]) <= TOL
    if nO == 0:
        assert np.array_equal(Y.view(np.uint16), o["Y"].view(np.uint16))

    # fp16-weight variant
    o16 = oracle.linear(X, Wq_h, sW_h, thr, stages=True, W16=W)
    acc16 = torch.empty((T, N), dtype=torch.int32, device=DEV)
    ws16 = li8.new_workspace(T, K, N, DEV)
    li8.prepare_fp16w(Xd, Wd, thr, ws16)
    Y16 = host(li8.gemm_fp16w(Wq, sW, Wd, T, ws16, acc=acc16))
    assert np.array_equal(host(acc16), o16["acc"])
    assert rel_err(Y16, o16["Y"]) <= TOL
    assert np.array_equal(Y16.view(np.uint16), host(li8.linear_fp16w(Xd, Wq, sW, Wd, thr)).view(np.uint16))

    # outlier-column cache: a miss, then a hit
    cache = li8.new_cache(K, N, DEV)
    for _ in range(2):
        Yc = host(li8.linear_cached(Xd, Wq, sW, cache, thr))
        assert np.array_equal(Yc.view(np.uint16), Y.view(np.uint16))

    # SmoothQuant-style W8A8 (calibrated on the batch itself)
    s = oracle.sq_factors(oracle.column_absmax(X), oracle.column_absmax(W), 0.5)
    Wq_s, sW_s = oracle.sq_quantize_weight(W, s)
    Ys = host(li8.smoothquant_linear(Xd, dev(np.float32(1.0) / s), dev(Wq_s), dev(sW_s)))
    assert np.array_equal(Ys.view(np.uint16), oracle.sq_linear(X, s, Wq_s, sW_s).view(np.uint16))
