"""llm_int8_linear_noalloc: the allocation-free linear, through the C ABI.

It runs the same kernels as llm_int8_linear with the library's fixed
per-GPU scratch array as the workspace, so its output must equal
llm_int8_linear's bit for bit (and so meet the oracle's bar, checked here
too on the small case).  Calls follow one another on one array, each
smaller than the last, so that a value left behind by an earlier call that
a later one relied on would show.
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


def case(name, **shape):
    X, W, _ = workloads.make(name, **shape)
    Xd = dev(X)
    Wq, sW = li8.quantize_weight(dev(W))
    return X, Xd, Wq, sW


def test_noalloc_equals_linear_on_successive_calls():
    # largest first: 4096 x 4096 x 11008 (about 96 MB of the 128 MiB array),
    # then a smaller tiled call with hundreds of outlier columns, a
    # few-token call (no scratch used) and a small tiled call again
    big = case("prefill_7b_ffn_up_t4096")
    mid = case("ffn_13b", T=300, K=1040, N=520, sparse_rate=2e-3)
    few = case("decode_7b_attn")
    small = case("tiny", T=40, K=64, N=96)
    calls = [("4096x4096x11008", big, 6.0), ("300x1040x520", mid, 6.0),
             ("8x4096x4096", few, 6.0), ("40x64x96", small, 6.0),
             ("300x1040x520 thr inf", mid, float("inf"))]
    outs = {}
    for label, (X, Xd, Wq, sW), thr in calls:
        print(f"case noalloc {label}", flush=True)
        T, N = X.shape[0], Wq.shape[0]
        ref = host(li8.linear(Xd, Wq, sW, thr))
        out = torch.empty((T, N), dtype=torch.float16, device=DEV)
        y = host(li8.linear_noalloc(Xd, Wq, sW, thr, out=out))
        assert np.array_equal(y.view(np.uint16), ref.view(np.uint16)), label
        outs[label] = y
    # the small case against the oracle as well
    X, Xd, Wq, sW = mid
    o = oracle.linear(X, host(Wq), host(sW), 6.0)
    y = outs["300x1040x520"].astype(np.float64)
    err = float(np.max(np.abs(y - o.astype(np.float64)) / (1 + np.abs(o.astype(np.float64)))))
    assert err <= TOL, err


def test_noalloc_allocates_nothing():
    """After the first call on the device (which looks up the array), calls
    leave the device's free memory unchanged."""
    X, Xd, Wq, sW = case("prefill_7b_ffn_up", T=1024)
    out = torch.empty((X.shape[0], Wq.shape[0]), dtype=torch.float16, device=DEV)
    li8.linear_noalloc(Xd, Wq, sW, 6.0, out=out)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for _ in range(3):
        li8.linear_noalloc(Xd, Wq, sW, 6.0, out=out)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free0


def test_noalloc_refuses_shapes_past_the_array():
    """The 70B slice needs more workspace than the array holds: refused on
    the host, nothing launched."""
    T, K, N = 4096, 8192, 28672
    assert li8.linear_workspace_bytes(T, K, N) > li8.NOALLOC_SCRATCH_BYTES
    X = torch.zeros((T, K), dtype=torch.float16, device=DEV)
    Wq = torch.zeros((N, K), dtype=torch.int8, device=DEV)
    sW = torch.zeros(N, dtype=torch.float32, device=DEV)
    with pytest.raises(li8.Int8MatmulError, match="LI8_ERR_SCRATCH"):
        li8.linear_noalloc(X, Wq, sW, 6.0)
