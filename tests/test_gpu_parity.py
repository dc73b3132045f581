"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar: bit-exact for the outlier column set, the int8 codes, the fp32 scales
and the int32 accumulators; for the fp16 output
max |Y_gpu - Y_oracle| / (1 + |Y_oracle|) <= 1e-2; with no outlier column
the output is bit-exact as well (both sides compute
fp16(fl32(fl32(acc * sX) * sW)) with no other term).

Every case is compared element by element (the full-size workloads are in
test_gpu_full_size.py).
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
    li8.load_library()  # raises if the HIP library is not built


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def say(msg):
    print(msg, flush=True)


def rel_err(y, ref):
    y = y.astype(np.float64)
    ref = ref.astype(np.float64)
    return float(np.max(np.abs(y - ref) / (1.0 + np.abs(ref)))) if y.size else 0.0


def bits_to_flags(words, K):
    w = words.view(np.uint32)
    j = np.arange(K)
    return ((w[j // 32] >> (j % 32).astype(np.uint32)) & 1).astype(np.uint8)


def gpu_run(X, W, thr):
    """Every stage of the HIP path for one call, copied back to the host."""
    T, K = X.shape
    N = W.shape[0]
    Xd, Wd = dev(X), dev(W)
    Wq, sW = li8.quantize_weight(Wd)
    ws = li8.new_workspace(T, K, N, DEV)
    li8.prepare(Xd, Wq, thr, ws)
    st = li8.export_stages(ws, T, K, N)
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    Y = li8.gemm(Wq, sW, T, ws, acc=acc)
    Yf = li8.linear(Xd, Wq, sW, thr)
    r = {k: host(v) for k, v in st.items()}
    r.update(Wq=host(Wq), sW=host(sW), acc=host(acc), Y=host(Y), Y_fused=host(Yf))
    return r


def chunks_to_rows(flat, T, nO):
    """[T, round_up(nO, 16)] from the 16-column chunk layout of the gathered
    outlier values: rank i of row t at ((i // 16) * T + t) * 16 + i % 16."""
    n16 = (nO + 15) // 16 * 16
    out = np.zeros((T, n16), dtype=flat.dtype)
    for c in range(n16 // 16):
        out[:, 16 * c:16 * c + 16] = flat[c * T * 16:(c + 1) * T * 16].reshape(T, 16)
    return out


def check_full(X, W, thr, label):
    say(f"case {label}: T={X.shape[0]} K={X.shape[1]} N={W.shape[0]} thr={thr}")
    T, K = X.shape
    g = gpu_run(X, W, thr)
    Wq, sW = oracle.quantize_weight(W)
    assert np.array_equal(g["Wq"], Wq), "weight codes"
    assert np.array_equal(g["sW"], sW), "weight scales"
    o = oracle.linear(X, Wq, sW, thr, stages=True)
    nO = int(g["n_outliers"][0])
    assert nO == o["nO"], "outlier count"
    assert np.array_equal(bits_to_flags(g["outlier_bits"], K), o["flags"]), "outlier set"
    assert np.array_equal(g["outlier_idx"][:nO], o["idx"]), "outlier index list"
    assert np.array_equal(g["Xq"], o["Xq"]), "token codes"
    assert np.array_equal(g["sX"][:T], o["sX"]), "token scales"
    XO = chunks_to_rows(g["X_out"], T, nO)
    assert np.array_equal(XO[:, :nO], X[:, o["idx"]]), "gathered outlier columns"
    assert np.all(XO[:, nO:].view(np.uint16) == 0), "zero pad of the gather"
    assert np.array_equal(g["acc"], o["acc"]), "int32 accumulators"
    assert np.array_equal(g["Y"].view(np.uint16), g["Y_fused"].view(np.uint16)), \
        "prepare+gemm and the fused call differ"
    e = rel_err(g["Y"], o["Y"])
    assert e <= TOL, f"fp16 output error {e}"
    if nO == 0:
        assert_bit_exact(g["Y"], o["Y"], g["acc"], o["sX"], sW)
    return g, o


def assert_bit_exact(yg, yo, acc, sX, sW):
    """With no outlier column both sides compute fp16(fl32(fl32(acc*sX)*sW))."""
    bad = np.argwhere(yg.view(np.uint16) != yo.view(np.uint16))
    if len(bad):
        lines = []
        for t, n in bad[:8]:
            lines.append(f"[{t},{n}] gpu={yg[t, n]!r} ({yg[t, n].view(np.uint16):#06x}) "
                         f"oracle={yo[t, n]!r} ({yo[t, n].view(np.uint16):#06x}) "
                         f"acc={acc[t, n]} sX={sX[t]!r} sW={sW[n]!r}")
        raise AssertionError(f"no outliers: {len(bad)} of {yg.size} outputs differ:\n"
                             + "\n".join(lines))


def with_outliers(X, cols, value):
    X = X.copy()
    X[:, cols] = np.float16(value)
    return X


# ---------------------------------------------------------------------------
# small shapes, element by element
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("thr", [6.0, 0.0, np.inf])
def test_tiny_workload(thr):
    X, W, _ = workloads.make("tiny")
    check_full(X, W, thr, f"tiny thr={thr}")


@pytest.mark.parametrize("T,K,N", [
    (300, 272, 520),     # ragged in every dimension: 2 M-tiles, 2 K-stages + 16, 3 N-tiles
    (513, 1024, 769),
    (1, 16, 1),
    (1, 16, 300),
    (257, 48, 33),       # K not a multiple of 32: the last bit-set word is half used
    (64, 4096, 64),
])
@pytest.mark.parametrize("thr", [6.0, np.inf, 0.0])
def test_ragged_shapes(T, K, N, thr):
    w = workloads.WORKLOADS["tiny"]
    rng = np.random.default_rng(T * 7 + K * 3 + N)
    X, _ = workloads.make_activation(w, seed=int(rng.integers(1 << 30)), T=T, K=K)
    W = workloads.make_weight(w, seed=int(rng.integers(1 << 30)), N=N, K=K)
    check_full(X, W, thr, f"ragged {T}x{K}x{N}")


# T <= 16: the few-token shapes, decode-time projections of 7B-70B layers
# among them (the library's path for each is llm_int8_plan's choice).
@pytest.mark.parametrize("T,K,N", [
    (1, 4096, 4101),     # one token; the last 16-feature row group holds 5 features
    (3, 48, 17),         # K not a multiple of 64: the last MFMA k-step is part padding
    (8, 4112, 300),      # K just above 4096: two 8-column chunks of X per thread
    (16, 8192, 130),     # the largest few-token shape
    (15, 1024, 1),       # a single output feature
    (16, 16, 33),        # one 16-column block of K
    (9, 2048, 100),      # the first T past the 8-token bound
    (8, 8192, 70),       # 8 tokens, two chunks of X per thread, the largest K
    (8, 4096, 11008),    # 7B FFN up: 688 row groups, about three per workgroup
    (16, 5120, 13824),   # 13B FFN up at 16 tokens: 864 row groups
    (8, 11008, 4096),    # 7B FFN down: K past the few-token kernel's bound
    (1, 13824, 512),     # 13B FFN down, one token
    (16, 28672, 64),     # 70B FFN down width, 16 tokens
    # the separate MFMA waves (K <= 4096, one row group per workgroup) at
    # their limits, and just past the row-group limit
    (16, 4096, 4096),    # 256 row groups, the largest K, 16 tokens
    (5, 3008, 4000),     # 47 k-steps: shares of 5 and 6, a ragged last row group
    (8, 4096, 4112),     # 257 row groups: the register-weight path and its loop
])
@pytest.mark.parametrize("thr", [6.0, np.inf, 0.0])
def test_decode_shapes(T, K, N, thr):
    w = workloads.WORKLOADS["decode_7b_attn"]
    rng = np.random.default_rng(T * 11 + K * 5 + N)
    X, _ = workloads.make_activation(w, seed=int(rng.integers(1 << 30)), T=T, K=K)
    W = workloads.make_weight(w, seed=int(rng.integers(1 << 30)), N=N, K=K)
    check_full(X, W, thr, f"decode {T}x{K}x{N}")


def test_decode_many_outliers():
    """Several 32-column chunks of outliers spread over many bit-set words,
    on the few-token path."""
    w = workloads.WORKLOADS["ffn_13b"]
    import dataclasses
    w = dataclasses.replace(w, T=8, K=5120, N=200, sparse_rate=5e-3)
    X, _ = workloads.make_activation(w)
    W = workloads.make_weight(w)
    g, o = check_full(X, W, 6.0, "decode many outliers")
    assert o["nO"] > 150


@pytest.mark.parametrize("n_out", [250, 257])
def test_outlier_count_at_gather_capacity(n_out):
    """Hundreds of outlier columns on either side of a multiple of 16 (the
    gathered matrices are padded to one), spread over every 128-column K
    stage of the GEMM, including the ragged last one (K = 1040 = 8*128 + 16)."""
    T, K, N = 300, 1040, 520
    rng = np.random.default_rng(n_out)
    X = rng.standard_normal((T, K)).astype(np.float32)
    cols = np.sort(rng.choice(K - 16, n_out - 1, replace=False))
    cols = np.append(cols, K - 7)   # one in the last, partial stage
    X[:, cols] = rng.choice([-1.0, 1.0], (T, n_out)) * rng.uniform(20, 60, (T, n_out))
    X = X.astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    g, o = check_full(X, W, 6.0, f"{n_out} outlier columns")
    assert o["nO"] == n_out


@pytest.mark.parametrize("which", ["min", "min+1", "cap", "cap+1", "dense stage"])
def test_gemm_fold_capacity(which):
    """On 128-wide tiles, with more than 64 and at most 256 outlier columns,
    the tiled GEMM copies their weight columns out of the K stages it
    streams through LDS; otherwise the prepare kernel gathers them.  Both
    sides of each limit, the columns spread over K, one in the ragged last
    stage; and 100 columns in one 128-column stage, more than a stage's
    share of one copy per thread (512 / 128)."""
    T, K, N = 300, 1040, 520
    n_out = {"min": 64, "min+1": 65, "cap": 256, "cap+1": 257, "dense stage": 100}[which]
    assert li8.plan(T, K, N) == dict(path="tiled", tile_m=256, tile_n=128, fold_lo=64, fold_hi=256)
    rng = np.random.default_rng(9000 + n_out)
    X = rng.standard_normal((T, K)).astype(np.float32)
    if which == "dense stage":
        cols = np.sort(rng.choice(128, n_out - 1, replace=False) + 256)
    else:
        cols = np.sort(rng.choice(K - 16, n_out - 1, replace=False))
    cols = np.append(cols, K - 5)
    X[:, cols] = rng.choice([-1.0, 1.0], (T, n_out)) * rng.uniform(20, 60, (T, n_out))
    X = X.astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    g, o = check_full(X, W, 6.0, f"fold capacity: {n_out} outlier columns")
    assert o["nO"] == n_out


@pytest.mark.parametrize("T,N,tile_n", [(1000, 16300, 256), (1000, 8320, 192)])
def test_wide_tiles_gather(T, N, tile_n):
    """The 192- and 256-wide tiles never copy the weight's outlier columns
    themselves: with 40 outlier columns the prepare kernel gathers them."""
    K = 1040
    assert li8.plan(T, K, N) == dict(path="tiled", tile_m=256, tile_n=tile_n, fold_lo=0, fold_hi=0)
    rng = np.random.default_rng(9100 + tile_n)
    X = rng.standard_normal((T, K)).astype(np.float32)
    cols = np.append(np.sort(rng.choice(K - 16, 39, replace=False)), K - 5)
    X[:, cols] = rng.choice([-1.0, 1.0], (T, 40)) * rng.uniform(20, 60, (T, 40))
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    g, o = check_full(X.astype(np.float16), W, 6.0, f"wide tile {tile_n}: 40 outlier columns")
    assert o["nO"] == 40


@pytest.mark.parametrize("n_out", [32, 33, 256, 257, 513])
def test_few_token_outlier_list_capacity(n_out):
    """The few-token kernel lists up to 256 outlier columns in LDS and
    gathers the first 32 with all threads; counts on either side of both
    limits, spread over K with one in the last 16 columns."""
    T, K, N = 8, 2048, 100
    rng = np.random.default_rng(7000 + n_out)
    X = rng.standard_normal((T, K)).astype(np.float32)
    cols = np.sort(rng.choice(K - 16, n_out - 1, replace=False))
    cols = np.append(cols, K - 3)
    X[:, cols] = rng.choice([-1.0, 1.0], (T, n_out)) * rng.uniform(20, 60, (T, n_out))
    X = X.astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    g, o = check_full(X, W, 6.0, f"few-token {n_out} outlier columns")
    assert o["nO"] == n_out


def test_many_outliers_13b_like():
    """Hundreds of outlier columns (token-sparse outliers as in the 13B
    workload, at a higher rate) on a reduced shape."""
    w = workloads.WORKLOADS["ffn_13b"]
    import dataclasses
    w = dataclasses.replace(w, T=128, K=5120, N=640, sparse_rate=2e-3)
    X, _ = workloads.make_activation(w)
    W = workloads.make_weight(w)
    g, o = check_full(X, W, 6.0, "13b-like many outliers")
    assert o["nO"] > 500


def test_degenerate_inputs():
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((96, 64)) * 0.05).astype(np.float16)
    # all-zero activation: every scale 0, output 0
    X = np.zeros((40, 64), np.float16)
    g, _ = check_full(X, W, 6.0, "zero X")
    assert np.all(g["Y"] == 0)
    # one token whose only non-zero values are outliers: scale 0 for that row
    X = (rng.standard_normal((40, 64))).astype(np.float16)
    X[5, :] = 0
    X[5, 3] = 50.0
    check_full(X, W, 6.0, "row with only an outlier")
    # a weight row of zeros
    W2 = W.copy()
    W2[7, :] = 0
    check_full(X, W2, 6.0, "zero weight row")
    # values exactly at the threshold are not outliers
    X = with_outliers((rng.standard_normal((40, 64)) * 0.5).astype(np.float16), [1, 9], 6.0)
    g, o = check_full(X, W, 6.0, "exactly 6.0")
    assert o["nO"] == 0
    X[0, 9] = np.nextafter(np.float16(6.0), np.float16(10))
    g, o = check_full(X, W, 6.0, "just above 6.0")
    assert list(o["idx"]) == [9]
    # every column an outlier (threshold 0 on a dense X)
    X = (rng.standard_normal((40, 64)) + 0.01).astype(np.float16)
    X[X == 0] = 1.0
    g, o = check_full(X, W, 0.0, "all columns outliers")
    assert o["nO"] == 64


def test_worked_example_on_gpu(golden):
    g = golden("worked_example.txt")
    vals = np.array([float(v) for v in g["values"]] + [0.0] * 10, np.float16)
    codes = [int(c) for c in g["codes"]]
    Wq, sW = li8.quantize_weight(dev(vals[None, :]))
    assert list(host(Wq)[0, :6]) == codes
    ws = li8.new_workspace(1, 16, 1, DEV)
    li8.prepare(dev(vals[None, :]), Wq, float("inf"), ws)
    st = li8.export_stages(ws, 1, 16, 1)
    assert list(host(st["Xq"])[0, :6]) == codes


def test_empty_and_k0_calls():
    Wq = torch.zeros((4, 16), dtype=torch.int8, device=DEV)
    sW = torch.ones(4, dtype=torch.float32, device=DEV)
    X = torch.zeros((0, 16), dtype=torch.float16, device=DEV)
    Y = li8.linear(X, Wq, sW)
    assert tuple(Y.shape) == (0, 4)
    X = torch.randn(5, 0, device=DEV).half()
    Y = torch.full((5, 3), 7.0, dtype=torch.float16, device=DEV)
    li8.linear(X, torch.zeros((3, 0), dtype=torch.int8, device=DEV),
               torch.ones(3, device=DEV), out=Y)
    assert torch.all(Y == 0)


def test_determinism_and_canary():
    X, W, _ = workloads.make("tiny", T=700, N=600, K=512)
    Xd, Wd = dev(X), dev(W)
    Wq, sW = li8.quantize_weight(Wd)
    T, N = X.shape[0], W.shape[0]
    sentinel = 0x7BCD
    buf = torch.full((T * N + 4096,), sentinel, dtype=torch.int16, device=DEV)
    Y = buf[: T * N].view(torch.float16).view(T, N)
    ws = li8.new_workspace(T, 512, N, DEV)
    li8.linear(Xd, Wq, sW, 6.0, out=Y, workspace=ws)
    y1 = host(Y).copy()
    li8.linear(Xd, Wq, sW, 6.0, out=Y, workspace=ws)
    assert np.array_equal(host(Y).view(np.uint16), y1.view(np.uint16))
    assert np.all(host(buf[T * N:]) == sentinel)


@pytest.mark.parametrize("T,K,N", [
    (300, 1040, 520),     # tiled path, few detection strips
    (4096, 512, 300),     # tiled path, all 16 detection strips
    (2050, 1040, 300),    # one wave per token row, the last workgroup half past T
    (8, 4096, 300),       # few tokens (prepare + gemm route)
    (8, 11008, 300),      # few tokens, split K (prepare + gemm route)
])
def test_dirty_workspace(T, K, N):
    """A workspace's contents on entry do not matter: every byte set (a
    partial bit set read before it was written would flag every column)
    gives the same stages and output as a zeroed one, for linear and for
    prepare + gemm."""
    X, W, _ = workloads.make("prefill_7b_ffn_up", T=T, K=K, N=N)
    Xd, Wd = dev(X), dev(W)
    Wq, sW = li8.quantize_weight(Wd)
    out = {}
    for fill in (0, 255):
        ws = li8.new_workspace(T, K, N, DEV)
        ws.fill_(fill)
        Y = li8.linear(Xd, Wq, sW, 6.0, workspace=ws)
        ws.fill_(fill)
        li8.prepare(Xd, Wq, 6.0, ws)
        st = {k: host(v).copy() for k, v in li8.export_stages(ws, T, K, N).items()}
        Y2 = li8.gemm(Wq, sW, T, ws)
        out[fill] = (host(Y).copy(), host(Y2).copy(), st)
    say(f"case dirty workspace {T}x{K}x{N}: {int(out[0][2]['n_outliers'][0])} outlier columns")
    for a, b in zip(out[0][:2], out[255][:2]):
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    nO = int(out[0][2]["n_outliers"][0])
    assert int(out[255][2]["n_outliers"][0]) == nO
    for k in ("outlier_bits", "sX", "Xq"):
        assert np.array_equal(out[0][2][k], out[255][2][k]), k
    assert np.array_equal(out[0][2]["outlier_idx"][:nO], out[255][2]["outlier_idx"][:nO])
    assert np.array_equal(out[0][0].view(np.uint16), out[0][1].view(np.uint16))


@pytest.mark.parametrize("T,K,N", [(300, 1040, 520), (8, 4096, 300), (8, 11008, 300)])
def test_dirty_workspace_variants(T, K, N):
    """The fp16-weight, cached and SmoothQuant-style calls, too, give the
    same output from a workspace whose every byte is set as from a zeroed
    one (the cache itself starts empty, as after llm_int8_cache_reset)."""
    X, W, _ = workloads.make("prefill_7b_ffn_up", T=T, K=K, N=N)
    Xd, Wd = dev(X), dev(W)
    Wq, sW = li8.quantize_weight(Wd)
    s_f, s_inv = li8.smoothquant_factors(li8.smoothquant_column_absmax(Xd),
                                         li8.smoothquant_column_absmax(Wd), 0.5)
    Wq_s, sW_s = li8.smoothquant_quantize_weight(Wd, s_f)
    out = {}
    for fill in (0, 255):
        ys = []
        ws = li8.new_workspace(T, K, N, DEV)
        ws.fill_(fill)
        ys.append(li8.linear_fp16w(Xd, Wq, sW, Wd, 6.0, workspace=ws))
        ws.fill_(fill)
        cache = li8.new_cache(K, N, DEV)
        ys.append(li8.linear_cached(Xd, Wq, sW, cache, 6.0, workspace=ws))
        ws.fill_(fill)
        ys.append(li8.linear_cached(Xd, Wq, sW, cache, 6.0, workspace=ws))   # a hit
        ws.fill_(fill)
        ys.append(li8.smoothquant_linear(Xd, s_inv, Wq_s, sW_s, workspace=ws))
        out[fill] = [host(y).copy() for y in ys]
    say(f"case dirty workspace variants {T}x{K}x{N}")
    for a, b in zip(out[0], out[255]):
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


@pytest.mark.parametrize("T,K,N,tile_n", [
    (1000, 272, 16300, 256),   # 4 x 64 tiles of 256x256: exactly one round
    (1000, 272, 8320, 192),    # 4 x 44 tiles of 256x192, the last 64 features wide
    (300, 272, 520, 128),      # 2 x 5 tiles of 256x128
])
def test_tile_shapes_ragged(T, K, N, tile_n):
    """Each output tile shape of the tiled GEMM on ragged T and N, every
    element against the oracle (int8 path), and the fp16-weight variant's
    output and accumulators on the same tiles."""
    p = li8.plan(T, K, N)
    assert (p["path"], p["tile_m"], p["tile_n"]) == ("tiled", 256, tile_n)
    w = workloads.WORKLOADS["prefill_7b_ffn_up"]
    X, _ = workloads.make_activation(w, seed=5 + tile_n, T=T, K=K)
    W = workloads.make_weight(w, seed=6 + tile_n, N=N, K=K)
    g, o = check_full(X, W, 6.0, f"tile {tile_n}: {T}x{K}x{N}")
    assert o["nO"] > 0, "the case should have outlier columns"
    Xd, Wd = dev(X), dev(W)
    Wq, sW = li8.quantize_weight(Wd)
    ws = li8.new_workspace(T, K, N, DEV)
    Yh = li8.linear_fp16w(Xd, Wq, sW, Wd, 6.0, workspace=ws)
    li8.prepare_fp16w(Xd, Wd, 6.0, ws)
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    Yh2 = li8.gemm_fp16w(Wq, sW, Wd, T, ws, acc=acc)
    oh = oracle.linear(X, g["Wq"], g["sW"], 6.0, stages=True, W16=W)
    assert np.array_equal(host(acc), oh["acc"]), "fp16-weight accumulators"
    yh = host(Yh)
    assert np.array_equal(yh.view(np.uint16), host(Yh2).view(np.uint16))
    e = rel_err(yh, oh["Y"])
    assert e <= TOL, f"fp16-weight output error {e}"


def test_many_tokens_narrow():
    """A token count far past one grid round of every kernel (the detection
    grid's rows per workgroup, 65538 quantization workgroups, 512 row tiles
    of the GEMM) on a narrow layer, checked in full against the oracle."""
    T, K, N = 131072, 32, 48
    rng = np.random.default_rng(31)
    X = rng.standard_normal((T, K)).astype(np.float32)
    X[:, 5] = rng.choice([-1.0, 1.0], T) * rng.uniform(20, 60, T)   # one fixed outlier column
    X[T - 1, 30] = np.float32(40.0)                                   # and one in the last row only
    X = X.astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    g, o = check_full(X, W, 6.0, "many tokens, narrow layer")
    assert o["nO"] == 2


# ---------------------------------------------------------------------------
# Long prompts (from 2048 tokens): with K <= 4096 the token quantization runs
# one wave per row, four rows per workgroup, and a ragged token count leaves
# the last workgroup's waves partly past T; a longer K keeps the workgroup per
# row.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,K,N", [
    (2048, 4096, 64),    # one wave per row, 8 chunks per lane
    (2051, 4112, 40),    # K past 4096: a workgroup per row
    (2050, 272, 520),    # 34 chunks per row: most lanes hold none; last workgroup half past T
    (8201, 1040, 48),    # 2051 workgroups of rows, the last with one live wave
    (4096, 8192, 32),    # the 70B slice's K
    (2049, 16, 40),      # one bit-set word, two chunks per row
    (2048, 4080, 24),    # the last bit-set word half used
])
@pytest.mark.parametrize("thr", [6.0, np.inf, 0.0])
def test_long_prompt_rows(T, K, N, thr):
    w = workloads.WORKLOADS["ffn_13b"]
    rng = np.random.default_rng(T + 5 * K + 7 * N)
    X, _ = workloads.make_activation(w, seed=int(rng.integers(1 << 30)), T=T, K=K)
    W = workloads.make_weight(w, seed=int(rng.integers(1 << 30)), N=N, K=K)
    check_full(X, W, thr, f"long prompt {T}x{K}x{N}")


def test_long_prompt_special_rows():
    """Rows whose scale is 0 (all zero; only outlier values) and many
    outlier columns spread over K, on the one-wave-per-row path (the last
    row, 2049, is the second wave of the last workgroup, whose other two
    waves are past T)."""
    T, K, N = 2050, 4096, 48
    rng = np.random.default_rng(41)
    X = np.clip(rng.standard_normal((T, K)), -5.0, 5.0).astype(np.float32)
    cols = np.sort(rng.choice(K, 300, replace=False))
    X[rng.integers(4, T - 1, 300), cols] = rng.choice([-1.0, 1.0], 300) * rng.uniform(7, 60, 300)
    X[3, :] = 0.0
    X[2049, :] = 0.0
    X[2049, cols[:5]] = 25.0
    X = X.astype(np.float16)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float16)
    g, o = check_full(X, W, 6.0, "long prompt, zero-scale rows, 300 outlier columns")
    assert o["nO"] == 300
    assert g["sX"][3] == 0 and g["sX"][2049] == 0


# ---------------------------------------------------------------------------
# llm_int8_stages: every intermediate result of one call, on each path
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,K,N", [
    (300, 272, 520),     # tiled path
    (8, 4096, 300),      # few tokens (two-call route of the fused kernel)
    (8, 11008, 300),     # few tokens, long K (split-K route)
    (2050, 1024, 96),    # one wave per token row in the prepare kernel
])
@pytest.mark.parametrize("thr", [6.0, np.inf, 0.0])
def test_stages_entry_point(T, K, N, thr):
    say(f"case stages {T}x{K}x{N} thr={thr}")
    w = workloads.WORKLOADS["ffn_13b"]
    rng = np.random.default_rng(T * 3 + K * 5 + N * 7)
    X, _ = workloads.make_activation(w, seed=int(rng.integers(1 << 30)), T=T, K=K)
    W = workloads.make_weight(w, seed=int(rng.integers(1 << 30)), N=N, K=K)
    Xd = dev(X)
    Wq, sW = li8.quantize_weight(dev(W))
    r = {k: host(v) for k, v in li8.stages(Xd, Wq, sW, thr).items()}
    Yl = host(li8.linear(Xd, Wq, sW, thr))
    o = oracle.linear(X, host(Wq), host(sW), thr, stages=True)
    nO = int(r["n_outliers"][0])
    assert nO == o["nO"], "outlier count"
    assert np.array_equal(r["flags"][:K], o["flags"]), "outlier flags"
    assert np.array_equal(r["outlier_idx"][:nO], o["idx"]), "outlier index list"
    assert np.array_equal(r["Xq"], o["Xq"]), "token codes"
    assert np.array_equal(r["sX"][:T], o["sX"]), "token scales"
    assert np.array_equal(r["X_out"][:, :nO], X[:, o["idx"]]), "gathered outlier values"
    assert np.array_equal(r["acc"], o["acc"]), "int32 accumulators"
    assert np.array_equal(r["Y"].view(np.uint16), Yl.view(np.uint16)), "stages and linear differ"
    e = rel_err(r["Y"], o["Y"])
    assert e <= TOL, f"fp16 output error {e}"
