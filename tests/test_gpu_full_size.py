"""Full-tensor parity at the full workload sizes, through the C ABI.

Every element of every stage is compared with the CPU oracle on the
seeded workloads (workloads/), at the shapes and in the launch
configuration the benchmark times:
  - the outlier set (bit set, count, ascending index list), the token codes
    Xq, the token scales sX, the gathered outlier values and the int32
    accumulators: bit-exact;
  - the fp16 output Y: max |Y_gpu - Y_oracle| / (1 + |Y_oracle|) <= 1e-2,
    and bit-exact when the call has no outlier column;
  - the one-call entry point against the two-call route (prepare + gemm):
    bit-identical Y.
The int8 path (llm_int8_linear), the fp16-weight variant
(llm_int8_linear_fp16w) and the SmoothQuant-style path (smoothquant_linear,
whose output is bit-exact since it has no floating-point sum) are covered.
"""
import gc

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


@pytest.fixture(autouse=True)
def _free():
    yield
    gc.collect()
    torch.cuda.empty_cache()


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


def chunks_to_rows(flat, T, nO):
    """[T, round_up(nO, 16)] from the 16-column chunk layout of the gathered
    outlier values: rank i of row t at ((i // 16) * T + t) * 16 + i % 16."""
    n16 = (nO + 15) // 16 * 16
    out = np.zeros((T, n16), dtype=flat.dtype)
    for c in range(n16 // 16):
        out[:, 16 * c:16 * c + 16] = flat[c * T * 16:(c + 1) * T * 16].reshape(T, 16)
    return out


def first_diff(a, b):
    bad = np.argwhere(a != b)
    return f"{len(bad)} differ, first at {tuple(bad[0])}" if len(bad) else ""


def check_stages(st, o, X, label):
    """The prepare stages against the oracle's, every element."""
    T, K = X.shape
    nO = int(host(st["n_outliers"])[0])
    assert nO == o["nO"], f"{label}: outlier count {nO} != {o['nO']}"
    assert np.array_equal(bits_to_flags(host(st["outlier_bits"]), K), o["flags"]), \
        f"{label}: outlier set"
    assert np.array_equal(host(st["outlier_idx"])[:nO], o["idx"]), f"{label}: index list"
    Xq = host(st["Xq"])
    assert np.array_equal(Xq, o["Xq"]), f"{label}: token codes, {first_diff(Xq, o['Xq'])}"
    sX = host(st["sX"])[:T]
    assert np.array_equal(sX.view(np.uint32), o["sX"].view(np.uint32)), f"{label}: token scales"
    XO = chunks_to_rows(host(st["X_out"]), T, nO)
    assert np.array_equal(XO[:, :nO].view(np.uint16), X[:, o["idx"]].view(np.uint16)), \
        f"{label}: gathered outlier values"
    assert np.all(XO[:, nO:].view(np.uint16) == 0), f"{label}: zero pad of the gather"
    return nO


def check_output(Y, Y2, o, nO, label):
    y, y2 = host(Y), host(Y2)
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16)), \
        f"{label}: the one-call and two-call routes differ"
    e = rel_err(y, o["Y"])
    assert e <= TOL, f"{label}: fp16 output error {e}"
    if nO == 0:
        d = first_diff(y.view(np.uint16), o["Y"].view(np.uint16))
        assert not d, f"{label}: no outliers, yet the output is not bit-exact: {d}"
    return e


INT8_FULL = ["tiny", "decode_7b_attn", "decode_7b_ffn_up", "decode_7b_ffn_down",
             "decode_13b_ffn_up", "decode_13b_ffn_down", "decode_70b_ffn_down",
             "prefill_7b_ffn_up", "prefill_7b_ffn_up_t4096", "ffn_13b",
             "ffn_70b_slice", "ffn_70b_slice_no_outliers"]


@pytest.mark.parametrize("name", INT8_FULL)
def test_int8_path_full(name):
    w = workloads.WORKLOADS[name]
    T, K, N = w.T, w.K, w.N
    label = f"full int8 {name} {T}x{K}x{N}"
    say(f"case {label}")
    X, W, cols = workloads.make(name)
    Xd, Wd = dev(X), dev(W)
    Wq, sW = li8.quantize_weight(Wd)
    del Wd
    ws = li8.new_workspace(T, K, N, DEV)
    Y = li8.linear(Xd, Wq, sW, w.threshold, workspace=ws)   # the call the benchmark times
    li8.prepare(Xd, Wq, w.threshold, ws)
    st = li8.export_stages(ws, T, K, N)
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    Y2 = li8.gemm(Wq, sW, T, ws, acc=acc)
    Wq_o, sW_o = oracle.quantize_weight(W)
    assert np.array_equal(host(Wq), Wq_o), f"{label}: weight codes"
    assert np.array_equal(host(sW).view(np.uint32), sW_o.view(np.uint32)), f"{label}: weight scales"
    o = oracle.linear(X, Wq_o, sW_o, w.threshold, stages=True)
    nO = check_stages(st, o, X, label)
    assert set(cols) <= set(o["idx"])
    a = host(acc)
    assert np.array_equal(a, o["acc"]), f"{label}: int32 accumulators, {first_diff(a, o['acc'])}"
    e = check_output(Y, Y2, o, nO, label)
    say(f"  {label}: nO={nO} max rel err {e:.3e}")


FP16W_FULL = ["decode_7b_attn", "decode_7b_ffn_down", "decode_13b_ffn_up",
              "prefill_7b_ffn_up_t4096", "ffn_13b"]


@pytest.mark.parametrize("name", FP16W_FULL)
def test_fp16_weight_variant_full(name):
    w = workloads.WORKLOADS[name]
    T, K, N = w.T, w.K, w.N
    label = f"full fp16w {name} {T}x{K}x{N}"
    say(f"case {label}")
    X, W, _ = workloads.make(name)
    Xd, Wd = dev(X), dev(W)
    Wq, sW = li8.quantize_weight(Wd)
    ws = li8.new_workspace(T, K, N, DEV)
    Y = li8.linear_fp16w(Xd, Wq, sW, Wd, w.threshold, workspace=ws)
    li8.prepare_fp16w(Xd, Wd, w.threshold, ws)
    st = li8.export_stages(ws, T, K, N)
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    Y2 = li8.gemm_fp16w(Wq, sW, Wd, T, ws, acc=acc)
    Wq_o, sW_o = oracle.quantize_weight(W)
    o = oracle.linear(X, Wq_o, sW_o, w.threshold, stages=True, W16=W)
    nO = check_stages(st, o, X, label)
    a = host(acc)
    assert np.array_equal(a, o["acc"]), f"{label}: int32 accumulators, {first_diff(a, o['acc'])}"
    e = check_output(Y, Y2, o, nO, label)
    say(f"  {label}: nO={nO} max rel err {e:.3e}")


SQ_FULL = ["decode_7b_attn", "decode_7b_ffn_down", "prefill_7b_ffn_up",
           "prefill_7b_ffn_up_t4096", "ffn_13b"]


@pytest.mark.parametrize("name", SQ_FULL)
def test_smoothquant_full(name):
    """Factors from 256 calibration rows drawn after X (alpha 0.5)."""
    w = workloads.WORKLOADS[name]
    T, K, N = w.T, w.K, w.N
    label = f"full sq {name} {T}x{K}x{N}"
    say(f"case {label}")
    Tcal = 256
    Xall, _ = workloads.make_activation(w, T=T + Tcal)
    X, Xcal = Xall[:T], Xall[T:]
    W = workloads.make_weight(w)
    s_o = oracle.sq_factors(oracle.column_absmax(Xcal), oracle.column_absmax(W), 0.5)
    Wq_o, sW_o = oracle.sq_quantize_weight(W, s_o)
    Wd = dev(W)
    s_g, r_g = li8.smoothquant_factors(li8.smoothquant_column_absmax(dev(Xcal)),
                                       li8.smoothquant_column_absmax(Wd), 0.5)
    Wq, sW = li8.smoothquant_quantize_weight(Wd, s_g)
    del Wd
    assert np.array_equal(host(s_g).view(np.uint32), s_o.view(np.uint32)), f"{label}: factors"
    assert np.array_equal(host(Wq), Wq_o), f"{label}: weight codes"
    assert np.array_equal(host(sW).view(np.uint32), sW_o.view(np.uint32)), f"{label}: weight scales"
    Xd = dev(X)
    ws = li8.new_workspace(T, K, N, DEV)
    Y = li8.smoothquant_linear(Xd, r_g, Wq, sW, workspace=ws)
    li8.smoothquant_prepare(Xd, r_g, N, ws)
    st = li8.export_stages(ws, T, K, N)
    acc = torch.empty((T, N), dtype=torch.int32, device=DEV)
    Y2 = li8.gemm(Wq, sW, T, ws, acc=acc)
    o = oracle.sq_linear(X, s_o, Wq_o, sW_o, stages=True)
    assert int(host(st["n_outliers"])[0]) == 0, f"{label}: no outlier columns"
    Xq = host(st["Xq"])
    assert np.array_equal(Xq, o["Xq"]), f"{label}: token codes, {first_diff(Xq, o['Xq'])}"
    assert np.array_equal(host(st["sX"])[:T].view(np.uint32), o["sX"].view(np.uint32)), \
        f"{label}: token scales"
    a = host(acc)
    assert np.array_equal(a, o["acc"]), f"{label}: int32 accumulators, {first_diff(a, o['acc'])}"
    y, y2 = host(Y), host(Y2)
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16)), f"{label}: routes differ"
    d = first_diff(y.view(np.uint16), o["Y"].view(np.uint16))
    assert not d, f"{label}: output not bit-exact: {d}"
    say(f"  {label}: bit-exact")
