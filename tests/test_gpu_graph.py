"""Calls captured in a HIP graph and replayed, and calls on two streams.

The calls allocate nothing given a workspace, never synchronize and read
no device state they have not written in the same call (no memset nodes),
so a captured call must give the eager call's output on every replay.  Each case
captures one call, replays it several times with eager work on the same
buffers in between (other inputs through the same workspace), and checks
every replay bit for bit against the eager output.  Shapes cover the tiled
path and the fused few-token kernel.
"""
import dataclasses

import numpy as np
import pytest
import torch

import int8_matmul_amd as li8
import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    li8.load_library()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def inputs(T, K, N, seed):
    w = dataclasses.replace(workloads.WORKLOADS["ffn_13b"], T=T, K=K, N=N, sparse_rate=2e-3)
    X, _ = workloads.make_activation(w, seed=seed)
    X2, _ = workloads.make_activation(w, seed=seed + 1)
    W = workloads.make_weight(w, seed=seed)
    return dev(X), dev(X2), dev(W)


def replay_and_check(call, disturb, out):
    """Eager reference, capture, then replays with `disturb` (eager calls
    through the same workspace) between them."""
    torch.cuda.synchronize()
    call()
    torch.cuda.synchronize()
    ref = out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on the capture stream
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(REPLAYS):
        out.zero_()
        disturb()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {i} differs from the eager call"


@pytest.mark.parametrize("T,K,N", [(300, 1024, 520), (8, 4096, 300), (16, 2048, 130)])
def test_linear_in_a_graph(T, K, N):
    print(f"case graph linear {T}x{K}x{N}", flush=True)
    X, X2, W = inputs(T, K, N, 11)
    Wq, sW = li8.quantize_weight(W)
    ws = li8.new_workspace(T, K, N, DEV)
    Y = torch.empty((T, N), dtype=torch.float16, device=DEV)
    Y2 = torch.empty_like(Y)
    replay_and_check(lambda: li8.linear(X, Wq, sW, 6.0, out=Y, workspace=ws),
                     lambda: li8.linear(X2, Wq, sW, 6.0, out=Y2, workspace=ws), Y)


@pytest.mark.parametrize("T,K,N", [(300, 1024, 520), (8, 4096, 300)])
def test_prepare_gemm_and_fp16w_in_a_graph(T, K, N):
    print(f"case graph prepare+gemm, fp16w {T}x{K}x{N}", flush=True)
    X, X2, W = inputs(T, K, N, 12)
    Wq, sW = li8.quantize_weight(W)
    ws = li8.new_workspace(T, K, N, DEV)
    Y = torch.empty((T, N), dtype=torch.float16, device=DEV)
    Y2 = torch.empty_like(Y)

    def two_halves():
        li8.prepare(X, Wq, 6.0, ws)
        li8.gemm(Wq, sW, T, ws, out=Y)

    replay_and_check(two_halves, lambda: li8.linear(X2, Wq, sW, 6.0, out=Y2, workspace=ws), Y)
    replay_and_check(lambda: li8.linear_fp16w(X, Wq, sW, W, 6.0, out=Y, workspace=ws),
                     lambda: li8.linear_fp16w(X2, Wq, sW, W, 6.0, out=Y2, workspace=ws), Y)


@pytest.mark.parametrize("T,K,N", [(300, 1024, 520), (8, 4096, 300)])
def test_smoothquant_in_a_graph(T, K, N):
    print(f"case graph smoothquant {T}x{K}x{N}", flush=True)
    X, X2, W = inputs(T, K, N, 13)
    s, s_inv = li8.smoothquant_factors(li8.smoothquant_column_absmax(X),
                                       li8.smoothquant_column_absmax(W), 0.5)
    Wq, sW = li8.smoothquant_quantize_weight(W, s)
    ws = li8.new_workspace(T, K, N, DEV)
    Y = torch.empty((T, N), dtype=torch.float16, device=DEV)
    Y2 = torch.empty_like(Y)
    replay_and_check(lambda: li8.smoothquant_linear(X, s_inv, Wq, sW, out=Y, workspace=ws),
                     lambda: li8.smoothquant_linear(X2, s_inv, Wq, sW, out=Y2, workspace=ws), Y)


@pytest.mark.parametrize("T,K,N", [(300, 1024, 520), (8, 4096, 300)])
def test_two_streams_two_workspaces(T, K, N):
    """Two calls in flight at once on two streams, each with its own
    workspace (the contract for concurrent calls), give the eager results."""
    print(f"case two streams {T}x{K}x{N}", flush=True)
    X, X2, W = inputs(T, K, N, 14)
    Wq, sW = li8.quantize_weight(W)
    ref1 = li8.linear(X, Wq, sW, 6.0)
    ref2 = li8.linear(X2, Wq, sW, 6.0)
    torch.cuda.synchronize()
    ws1, ws2 = li8.new_workspace(T, K, N, DEV), li8.new_workspace(T, K, N, DEV)
    Y1 = torch.empty((T, N), dtype=torch.float16, device=DEV)
    Y2 = torch.empty_like(Y1)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for _ in range(3):
        Y1.zero_()
        Y2.zero_()
        s1.wait_stream(torch.cuda.current_stream())
        s2.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s1):
            for _ in range(4):
                li8.linear(X, Wq, sW, 6.0, out=Y1, workspace=ws1)
        with torch.cuda.stream(s2):
            for _ in range(4):
                li8.linear(X2, Wq, sW, 6.0, out=Y2, workspace=ws2)
        torch.cuda.synchronize()
        assert torch.equal(Y1.view(torch.int16), ref1.view(torch.int16))
        assert torch.equal(Y2.view(torch.int16), ref2.view(torch.int16))
