"""The outlier-column cache (llm_int8_*_cached).

The pages note that the outlier features sit on the same few channels from
token to token (lowentro.cn "model quantization" notes, Q4), so the set of
outlier columns tends to repeat across calls; the cache keeps the outlier
columns of Wq gathered for the last set and skips that gather when the set
repeats.  Detection runs on every call, so the bar is: Y bit-identical to
llm_int8_linear on every call, whatever the cache holds, with the hit / miss
counters in the cache header telling which calls reused it.
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


def same_bits(a, b):
    return np.array_equal(host(a).view(np.uint16), host(b).view(np.uint16))


def batches(T, K, N, sparse=0.0, seed=0):
    """W and four activation batches: a, a with its rows permuted (same
    outlier set), b (other fixed columns) and a with one more outlier column."""
    w = dataclasses.replace(workloads.WORKLOADS["prefill_7b_ffn_up"], T=T, K=K, N=N,
                            sparse_rate=sparse, sp_lo=7.0, sp_hi=30.0)
    a, cols = workloads.make_activation(w, seed=seed)
    b, _ = workloads.make_activation(w, seed=seed + 100)
    W = workloads.make_weight(w, seed=seed)
    rng = np.random.default_rng(seed + 7)
    a_perm = a[rng.permutation(T)]
    a_more = a.copy()
    free = np.setdiff1d(np.arange(K), cols)
    a_more[T // 2, free[len(free) // 2]] = np.float16(50.0)
    return W, dict(a=a, a_perm=a_perm, b=b, a_more=a_more)


@pytest.mark.parametrize("T,K,N,sparse", [
    (300, 272, 520, 0.0),       # ragged tiles, a few fixed outlier columns
    (96, 2048, 384, 2e-3),      # hundreds of outlier columns spread over K
    (1000, 4096, 1100, 0.0),
    (1000, 272, 8320, 0.0),     # 256x192 GEMM tiles, the last 64 features wide
    (2050, 1024, 700, 2e-4),    # one wave per token row in the prepare kernel; 330 outlier columns
])
def test_sequence_hits_misses_and_bits(T, K, N, sparse):
    print(f"case cache sequence {T}x{K}x{N} sparse={sparse}", flush=True)
    W, xs = batches(T, K, N, sparse)
    Wq, sW = li8.quantize_weight(dev(W))
    cache = li8.new_cache(K, N, DEV)
    ws = li8.new_workspace(T, K, N, DEV)
    order = ["a", "a", "a_perm", "b", "b", "a_more", "a"]
    expect_hit = [False, True, True, False, True, False, False]
    hits = misses = 0
    for name, hit in zip(order, expect_hit):
        X = dev(xs[name])
        Yc = li8.linear_cached(X, Wq, sW, cache, 6.0, workspace=ws)
        Yu = li8.linear(X, Wq, sW, 6.0)
        assert same_bits(Yc, Yu), f"{name}: cached and uncached Y differ"
        hits += hit
        misses += not hit
        st = li8.cache_stats(cache)
        assert (st["hits"], st["misses"]) == (hits, misses), (name, st)
        assert st["valid"] == 1
    # the last call against the oracle (the uncached path is parity-tested
    # against it everywhere; this ties the cached one to it directly)
    o = oracle.linear(xs["a"], host(Wq), host(sW), 6.0, stages=True)
    assert st["nO"] == o["nO"]
    y = host(Yc).astype(np.float64)
    ref = o["Y"].astype(np.float64)
    assert float(np.max(np.abs(y - ref) / (1.0 + np.abs(ref)))) <= 1e-2


def test_halves_match_the_whole_call():
    W, xs = batches(300, 1024, 700)
    T, K, N = 300, 1024, 700
    Wq, sW = li8.quantize_weight(dev(W))
    cache = li8.new_cache(K, N, DEV)
    ws = li8.new_workspace(T, K, N, DEV)
    X = dev(xs["a"])
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    for _ in range(2):   # a miss, then a hit
        li8.prepare_cached(X, Wq, 6.0, ws, cache)
        Y2 = li8.gemm_cached(Wq, sW, T, ws, cache, acc=acc)
        Y = li8.linear(X, Wq, sW, 6.0)
        assert same_bits(Y, Y2)
        o = oracle.linear(xs["a"], host(Wq), host(sW), 6.0, stages=True)
        assert np.array_equal(host(acc), o["acc"])
    assert li8.cache_stats(cache)["hits"] == 1


def test_no_outliers_is_cached_too():
    W, xs = batches(300, 512, 300)
    Wq, sW = li8.quantize_weight(dev(W))
    cache = li8.new_cache(512, 300, DEV)
    X = dev(xs["a"])
    for _ in range(3):
        assert same_bits(li8.linear_cached(X, Wq, sW, cache, float("inf")),
                         li8.linear(X, Wq, sW, float("inf")))
    st = li8.cache_stats(cache)
    assert (st["valid"], st["nO"], st["hits"], st["misses"]) == (1, 0, 2, 1)


def test_few_tokens_leave_the_cache_alone():
    W, xs = batches(8, 4096, 300)
    Wq, sW = li8.quantize_weight(dev(W))
    cache = li8.new_cache(4096, 300, DEV)
    X = dev(xs["a"])
    ws = li8.new_workspace(8, 4096, 300, DEV)
    assert same_bits(li8.linear_cached(X, Wq, sW, cache, workspace=ws), li8.linear(X, Wq, sW))
    li8.prepare_cached(X, Wq, 6.0, ws, cache)
    assert same_bits(li8.gemm_cached(Wq, sW, 8, ws, cache), li8.linear(X, Wq, sW))
    st = li8.cache_stats(cache)
    assert (st["valid"], st["hits"], st["misses"]) == (0, 0, 0)


def test_reset_after_the_weight_changes_and_a_hit_reuses_the_columns():
    """A hit reads the cached columns instead of gathering: shown by handing
    the cache a different weight without a reset (outside the contract), which
    must give a different Y; after llm_int8_cache_reset the result is right.
    (Token-sparse outliers give more outlier columns than the GEMM copies out
    of its own K stages, at most 256, so the GEMM reads the cache's columns.)"""
    T, K, N = 256, 1024, 512
    W1, xs = batches(T, K, N, sparse=2e-3, seed=3)
    W2 = (W1.astype(np.float32) * -1.5).astype(np.float16)
    X = dev(xs["a"])
    Wq1, sW1 = li8.quantize_weight(dev(W1))
    Wq2, sW2 = li8.quantize_weight(dev(W2))
    cache = li8.new_cache(K, N, DEV)
    li8.linear_cached(X, Wq1, sW1, cache)
    assert li8.cache_stats(cache)["nO"] > 256
    stale = li8.linear_cached(X, Wq2, sW2, cache)
    assert li8.cache_stats(cache)["hits"] == 1
    assert not same_bits(stale, li8.linear(X, Wq2, sW2))
    li8.cache_reset(cache, K, N)
    assert li8.cache_stats(cache)["valid"] == 0
    assert same_bits(li8.linear_cached(X, Wq2, sW2, cache), li8.linear(X, Wq2, sW2))
    st = li8.cache_stats(cache)
    assert (st["hits"], st["misses"]) == (0, 1)


def test_graph_replays_hit():
    """Captured calls keep working (the cache logic is on the device)."""
    W, xs = batches(512, 2048, 1024)
    T, K, N = 512, 2048, 1024
    Wq, sW = li8.quantize_weight(dev(W))
    cache = li8.new_cache(K, N, DEV)
    ws = li8.new_workspace(T, K, N, DEV)
    X = dev(xs["a"])
    Y = torch.empty((T, N), dtype=torch.float16, device=DEV)
    ref = li8.linear(X, Wq, sW)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        li8.linear_cached(X, Wq, sW, cache, out=Y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        li8.linear_cached(X, Wq, sW, cache, out=Y, workspace=ws)
    for _ in range(3):
        Y.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert same_bits(Y, ref)
    st = li8.cache_stats(cache)
    assert st["misses"] == 1 and st["hits"] >= 3
