"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar: bit-exact for the outlier column set, the int8 codes, the fp32 scales
and the int32 accumulators; for the fp16 output
max |Y_gpu - Y_oracle| / (1 + |Y_oracle|) <= 1e-2; with no outlier column
the output is bit-exact as well (both sides compute
fp16(fl32(fl32(acc * sX) * sW)) with no other term).

Small shapes are compared element by element; the full-size workloads on
sampled rows (the outlier set is computed by the oracle over all of X).
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


# T <= 16 and K <= 8192 take the few-token path (one fused kernel for
# linear, a kernel reading the prepared workspace for gemm).
@pytest.mark.parametrize("T,K,N", [
    (1, 4096, 4101),     # one token; the last 16-feature row group holds 5 features
    (3, 48, 17),         # K not a multiple of 64: the last MFMA k-step is part padding
    (8, 4112, 300),      # K just above 4096: two 8-column chunks of X per thread
    (16, 8192, 130),     # the largest few-token shape
    (15, 1024, 1),       # a single output feature
    (16, 16, 33),        # one 16-column block of K
    (9, 2048, 100),      # the first T past the 8-token bound
    (8, 8192, 70),       # 8 tokens, two chunks of X per thread, the largest K
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


@pytest.mark.parametrize("n_out", [32, 33, 512, 513])
def test_few_token_outlier_list_capacity(n_out):
    """The few-token kernel lists up to 512 outlier columns in LDS and
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


def test_large_tile_ragged_sampled():
    """Ragged T and N where the 256x256 tiles fill exactly one round of
    workgroups (so the library keeps them), checked on sampled rows,
    accumulators included."""
    T, K, N = 1000, 272, 16300
    w = workloads.WORKLOADS["prefill_7b_ffn_up"]
    X, _ = workloads.make_activation(w, seed=5, T=T, K=K)
    W = workloads.make_weight(w, seed=6, N=N, K=K)
    say(f"case large-tile ragged: T={T} K={K} N={N}")
    Xd, Wd = dev(X), dev(W)
    Wq, sW = li8.quantize_weight(Wd)
    ws = li8.new_workspace(T, K, N, DEV)
    Y = li8.linear(Xd, Wq, sW, 6.0, workspace=ws)
    li8.prepare(Xd, Wq, 6.0, ws)
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    Y2 = li8.gemm(Wq, sW, T, ws, acc=acc)
    Wq_o, sW_o = oracle.quantize_weight(W)
    rows = np.array([0, 1, 255, 256, 511, 767, 768, 998, 999])
    Yo, idx, Xq_o, sX_o, acc_o = oracle.linear_rows(X, Wq_o, sW_o, 6.0, rows)
    rows_t = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(host(acc.index_select(0, rows_t)), acc_o)
    yg = host(Y.index_select(0, rows_t))
    assert np.array_equal(yg.view(np.uint16), host(Y2.index_select(0, rows_t)).view(np.uint16))
    e = rel_err(yg, Yo)
    assert e <= TOL, f"fp16 output error {e}"


def test_mid_tile_ragged_sampled():
    """Ragged T and N where 256x128 tiles would need a second round and
    256x256 tiles would leave a third of the round empty, so the library
    takes 256x192 tiles (4 x 44, the last 64 features wide): int8 and
    fp16-weight outlier products on sampled rows, accumulators included."""
    T, K, N = 1000, 272, 8320
    w = workloads.WORKLOADS["prefill_7b_ffn_up"]
    X, _ = workloads.make_activation(w, seed=7, T=T, K=K)
    W = workloads.make_weight(w, seed=8, N=N, K=K)
    say(f"case mid-tile ragged: T={T} K={K} N={N}")
    Xd, Wd = dev(X), dev(W)
    Wq, sW = li8.quantize_weight(Wd)
    ws = li8.new_workspace(T, K, N, DEV)
    Y = li8.linear(Xd, Wq, sW, 6.0, workspace=ws)
    Yh = li8.linear_fp16w(Xd, Wq, sW, Wd, 6.0, workspace=ws)
    li8.prepare(Xd, Wq, 6.0, ws)
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    Y2 = li8.gemm(Wq, sW, T, ws, acc=acc)
    Wq_o, sW_o = oracle.quantize_weight(W)
    rows = np.array([0, 1, 255, 256, 511, 767, 768, 998, 999])
    Yo, idx, Xq_o, sX_o, acc_o = oracle.linear_rows(X, Wq_o, sW_o, 6.0, rows)
    assert len(idx) > 0, "the case should have outlier columns"
    rows_t = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(host(acc.index_select(0, rows_t)), acc_o)
    yg = host(Y.index_select(0, rows_t))
    assert np.array_equal(yg.view(np.uint16), host(Y2.index_select(0, rows_t)).view(np.uint16))
    e = rel_err(yg, Yo)
    assert e <= TOL, f"fp16 output error {e}"
    Yho = oracle.linear_rows(X, Wq_o, sW_o, 6.0, rows, W16=W)[0]
    e = rel_err(host(Yh.index_select(0, rows_t)), Yho)
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
# full-size workloads, sampled rows
# ---------------------------------------------------------------------------

FULL = ["decode_7b_attn", "prefill_7b_ffn_up", "prefill_7b_ffn_up_t4096", "ffn_13b",
        "ffn_70b_slice", "ffn_70b_slice_no_outliers"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled(name):
    w = workloads.WORKLOADS[name]
    say(f"case full {name}: T={w.T} K={w.K} N={w.N}")
    X, W, cols = workloads.make(name)
    T, K, N = w.T, w.K, w.N
    Xd, Wd = dev(X), dev(W)
    Wq, sW = li8.quantize_weight(Wd)
    ws = li8.new_workspace(T, K, N, DEV)
    Y = li8.linear(Xd, Wq, sW, w.threshold, workspace=ws)   # the call the benchmark times
    li8.prepare(Xd, Wq, w.threshold, ws)   # the stages are defined by a prepare call
    st = li8.export_stages(ws, T, K, N)
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    Y2 = li8.gemm(Wq, sW, T, ws, acc=acc)
    Wq_o, sW_o = oracle.quantize_weight(W)
    assert np.array_equal(host(sW), sW_o)
    assert np.array_equal(host(Wq), Wq_o)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([[0, 1, T // 2, T - 1], rng.integers(0, T, 4)]))
    Yo, idx, Xq_o, sX_o, acc_o = oracle.linear_rows(X, Wq_o, sW_o, w.threshold, rows)
    nO = int(host(st["n_outliers"])[0])
    assert nO == len(idx) and np.array_equal(host(st["outlier_idx"])[:nO], idx)
    assert set(cols) <= set(idx)
    rows_t = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(host(st["Xq"].index_select(0, rows_t)), Xq_o)
    assert np.array_equal(host(st["sX"])[rows], sX_o)
    assert np.array_equal(host(acc.index_select(0, rows_t)), acc_o)
    yg = host(Y.index_select(0, rows_t))
    assert np.array_equal(yg.view(np.uint16), host(Y2.index_select(0, rows_t)).view(np.uint16))
    e = rel_err(yg, Yo)
    assert e <= TOL, f"{name}: fp16 output error {e}"
    if nO == 0:
        assert_bit_exact(yg, Yo, acc_o, sX_o, sW_o)
    say(f"  {name}: nO={nO} max rel err {e:.3e}")
