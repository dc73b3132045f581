"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each check is a value the
pages print, a closed form, an invariant, a special case that reduces to a
library routine (numpy), or a brute force written separately in pure
Python (oracle/brute.py).  All run on the CPU.
"""
import math

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import workloads
from oracle import brute

F16_6 = np.float16(6.0)
F16_6_UP = np.nextafter(np.float16(6.0), np.float16(np.inf))  # 6.00390625


def f16(a):
    return np.asarray(a, dtype=np.float16)


def ulp_distance(a16, b16):
    """Distance in binary16 units in the last place (same-sign finite values)."""
    a = a16.view(np.uint16).astype(np.int32)
    b = b16.view(np.uint16).astype(np.int32)
    # map sign-magnitude to a monotone integer line
    a = np.where(a & 0x8000, -(a & 0x7FFF), a)
    b = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(a - b)


# --------------------------------------------------------------------------
# binary16 conversion (the oracle writes its own)
# --------------------------------------------------------------------------

def test_h2d_all_bit_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    ours = oracle.h2d(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # sign of zero
    assert math.copysign(1.0, ours[0x8000]) == -1.0


def test_d2h_round_trip_and_ties_match_numpy():
    bits = np.arange(65536, dtype=np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    fin = np.isfinite(vals)
    assert np.array_equal(oracle.d2h(vals[fin]), bits[fin])
    # exact midpoints between neighbours (ties) and points just off them
    lo = np.arange(0, 0x7BFF, dtype=np.uint16).view(np.float16).astype(np.float64)
    hi = np.arange(1, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mid = (lo + hi) / 2  # exact in binary64
    with np.errstate(over="ignore"):
        for x in (mid, -mid, np.nextafter(mid, 0), np.nextafter(mid, np.inf)):
            assert np.array_equal(oracle.d2h(x), x.astype(np.float16).view(np.uint16))
        rng = np.random.default_rng(1)
        x = rng.standard_normal(200000) * np.exp(rng.uniform(-30, 12, 200000))
        assert np.array_equal(oracle.d2h(x), x.astype(np.float16).view(np.uint16))
        big = np.array([65504.0, 65519.99, 65520.0, 1e9, -65520.0])
        assert np.array_equal(oracle.d2h(big), big.astype(np.float16).view(np.uint16))


# --------------------------------------------------------------------------
# values the pages print
# --------------------------------------------------------------------------

def test_worked_example_weight_codes(golden):
    g = golden("worked_example.txt")
    vals = np.array([float(v) for v in g["values"]])
    codes = np.array([int(c) for c in g["codes"]], dtype=np.int8)
    W = f16(vals)[None, :]
    Wq, sW = oracle.quantize_weight(W)
    assert np.array_equal(Wq[0], codes)
    # the scale is max|W| / 127 of the fp16 values
    assert sW[0] == np.float32(np.float32(np.float16(8.9)) / np.float32(127))


def test_worked_example_as_activation_without_outliers(golden):
    """The same vector as a token row: with no outlier column (threshold
    above 8.9) the token scale is its absmax / 127 and the codes are the
    printed ones."""
    g = golden("worked_example.txt")
    vals = np.array([float(v) for v in g["values"]])
    codes = np.array([int(c) for c in g["codes"]], dtype=np.int8)
    X = f16(vals)[None, :]
    for thr in (np.inf, 9.0, 100.0):
        flags, idx = oracle.detect_outliers(X, thr)
        assert len(idx) == 0
        Xq, sX = oracle.quantize_rows(X, flags)
        assert np.array_equal(Xq[0], codes)
    # at threshold 6 the 8.9 column is an outlier: code 0 there, and the
    # row scale falls to 4.7/127 so -1.5 -> -41, 4.7 -> 127, -2.3 -> -62
    flags, idx = oracle.detect_outliers(X, 6.0)
    assert list(idx) == [4]
    Xq, sX = oracle.quantize_rows(X, flags)
    assert list(Xq[0]) == [0, -41, 127, 0, 0, -62]


def test_scale_example(golden):
    g = golden("scale_example.txt")
    amax = float(g["absmax"][0])
    approx = float(g["scale_approx"][0])
    digits = int(g["scale_printed_digits"][0])
    W = f16([[amax, -1.0, 0.5, 3.0]])
    _, sW = oracle.quantize_weight(W)
    assert round(float(sW[0]), digits) == approx
    assert sW[0] == np.float32(amax) / np.float32(127)


def test_outlier_damage_example(golden):
    g = golden("outlier_damage.txt")
    n = int(g["n_normal"][0])
    lo, hi = float(g["normal_lo"][0]), float(g["normal_hi"][0])
    out = float(g["outlier"][0])
    rng = np.random.default_rng(0)
    row = np.concatenate([rng.uniform(lo, hi, n), [out]])
    X = f16(row)[None, :]
    # one scale for the whole tensor (no decomposition): normal values crushed
    flags, idx = oracle.detect_outliers(X, np.inf)
    Xq, sX = oracle.quantize_rows(X, flags)
    assert sX[0] == np.float32(out) / np.float32(127)
    assert Xq[0, :n].min() >= 0 and Xq[0, :n].max() <= int(g["normal_codes_max"][0])
    assert Xq[0, n] == int(g["outlier_code"][0])
    # with the decomposition at threshold 6 the 100.0 column leaves the int8
    # product and the normal values use the whole code range again
    flags, idx = oracle.detect_outliers(X, 6.0)
    assert list(idx) == [n]
    Xq, sX = oracle.quantize_rows(X, flags)
    assert Xq[0, n] == 0
    assert Xq[0, :n].max() == 127
    assert len(np.unique(Xq[0, :n])) == 128  # codes 0..127 all in use


# --------------------------------------------------------------------------
# outlier detection: definition, boundary, monotonicity
# --------------------------------------------------------------------------

def test_detect_boundary_is_strict():
    X = f16([[0.0, F16_6, -F16_6, F16_6_UP, -F16_6_UP, 5.996, 1e4]])
    flags, idx = oracle.detect_outliers(X, 6.0)
    assert list(idx) == [3, 4, 6]
    assert list(flags) == [0, 0, 0, 1, 1, 0, 1]
    # threshold 0: every non-zero column, and a zero column never
    flags, idx = oracle.detect_outliers(X, 0.0)
    assert list(idx) == [1, 2, 3, 4, 5, 6]


def test_detect_brute_force_and_monotone():
    X, _, cols = workloads.make("tiny")
    xa = np.abs(X.astype(np.float64))
    prev = None
    for thr in [0.0, 0.5, 2.0, 4.0, 6.0, 20.0, 59.0, np.inf]:
        flags, idx = oracle.detect_outliers(X, thr)
        ref = np.nonzero((xa > thr).any(axis=0))[0]
        assert np.array_equal(idx, ref)
        assert np.array_equal(flags, (xa > thr).any(axis=0).astype(np.uint8))
        if prev is not None:
            assert set(idx) <= set(prev)  # higher threshold -> subset
        prev = idx
    flags, idx = oracle.detect_outliers(X, 6.0)
    assert set(cols) <= set(idx)


# --------------------------------------------------------------------------
# quantization: closed-form properties
# --------------------------------------------------------------------------

def test_absmax_maps_to_127_for_every_fp16_absmax():
    """The clip range reading: [-127,127] vs the page's clip(-128,127).  For
    every positive finite fp16 absmax a, fl32(a / fl32(a/127)) rounds to
    127, so -128 is never reached and both clip ranges give equal codes."""
    bits = np.arange(1, 0x7C00, dtype=np.uint16)
    a = bits.view(np.float16)
    W = np.stack([a, -a, np.zeros_like(a)], axis=1)  # [30719, 3]
    Wq, sW = oracle.quantize_weight(W)
    assert np.all(Wq[:, 0] == 127) and np.all(Wq[:, 1] == -127) and np.all(Wq[:, 2] == 0)
    assert np.array_equal(sW, a.astype(np.float32) / np.float32(127))


def test_quantize_invariants_on_workload():
    X, W, cols = workloads.make("tiny")
    Wq, sW = oracle.quantize_weight(W)
    flags, idx = oracle.detect_outliers(X, 6.0)
    Xq, sX = oracle.quantize_rows(X, flags)
    for q, src in ((Wq, W), (Xq, X)):
        assert np.abs(q.astype(np.int32)).max() <= 127
        s = np.sign(src.astype(np.float32))
        qs = np.sign(q)
        assert np.all((qs == 0) | (qs == s))
    # the absmax element of every weight row maps to +-127
    am = np.argmax(np.abs(W.astype(np.float32)), axis=1)
    assert np.all(np.abs(Wq[np.arange(W.shape[0]), am].astype(np.int32)) == 127)
    # outlier columns carry code 0; normal-column absmax maps to +-127
    assert np.all(Xq[:, idx] == 0)
    Xn = np.where(flags[None, :] == 1, 0, np.abs(X.astype(np.float32)))
    am = np.argmax(Xn, axis=1)
    assert np.all(np.abs(Xq[np.arange(X.shape[0]), am].astype(np.int32)) == 127)
    assert np.array_equal(sX, Xn.max(axis=1).astype(np.float32) / np.float32(127))


def test_power_of_two_row_scaling():
    """Scaling a token row by 2^k leaves its codes unchanged and scales its
    fp32 scale by exactly 2^k (no fp16 overflow/underflow in range)."""
    X, _, _ = workloads.make("tiny")
    X = X[:, :64].copy()
    X[np.abs(X) > 4] = 1.0
    flags = np.zeros(64, np.uint8)
    Xq, sX = oracle.quantize_rows(X, flags)
    for k in (-3, -1, 1, 2, 5):
        Y = (X.astype(np.float32) * np.float32(2.0 ** k)).astype(np.float16)
        Yq, sY = oracle.quantize_rows(Y, flags)
        assert np.array_equal(Yq, Xq)
        assert np.array_equal(sY, sX * np.float32(2.0 ** k))


def test_zero_rows_have_zero_scale_and_codes():
    X = np.zeros((3, 32), np.float16)
    X[1, 5] = 50.0  # a row whose only non-zero value is an outlier
    flags, idx = oracle.detect_outliers(X, 6.0)
    Xq, sX = oracle.quantize_rows(X, flags)
    assert list(idx) == [5]
    assert np.all(sX == 0) and np.all(Xq == 0)
    Wq, sW = oracle.quantize_weight(np.zeros((2, 16), np.float16))
    assert np.all(Wq == 0) and np.all(sW == 0)


# --------------------------------------------------------------------------
# the int8 product and the whole path: library routines and special cases
# --------------------------------------------------------------------------

def test_int8_gemm_matches_numpy_int64():
    rng = np.random.default_rng(3)
    A = rng.integers(-127, 128, (37, 300), dtype=np.int8)
    B = rng.integers(-127, 128, (29, 300), dtype=np.int8)
    acc = oracle.int8_gemm(A, B)
    ref = A.astype(np.int64) @ B.astype(np.int64).T
    assert np.array_equal(acc, ref.astype(np.int32))
    # extreme values: +-127 everywhere gives +-K*16129 exactly
    A = np.full((2, 4096), 127, np.int8)
    B = np.full((3, 4096), -127, np.int8)
    assert np.all(oracle.int8_gemm(A, B) == -4096 * 16129)


def _numpy_vectorwise_int8(X, W):
    """Independent numpy re-statement of plain vector-wise int8 matmul."""
    x = X.astype(np.float32)
    w = W.astype(np.float32)
    sx = (np.abs(x).max(axis=1) / np.float32(127)).astype(np.float32)
    sw = (np.abs(w).max(axis=1) / np.float32(127)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        qx = np.where(sx[:, None] > 0, np.clip(np.rint(x / sx[:, None]), -127, 127), 0)
        qw = np.where(sw[:, None] > 0, np.clip(np.rint(w / sw[:, None]), -127, 127), 0)
    acc = qx.astype(np.int64) @ qw.astype(np.int64).T
    d = acc.astype(np.float32) * sx[:, None]
    d = (d * sw[None, :]).astype(np.float32)
    return d.astype(np.float16), qx.astype(np.int8), acc


def test_threshold_inf_is_pure_vectorwise_int8():
    X, W, _ = workloads.make("tiny")
    Wq, sW = oracle.quantize_weight(W)
    r = oracle.linear(X, Wq, sW, np.inf, stages=True)
    assert r["nO"] == 0
    Yref, qx, acc = _numpy_vectorwise_int8(X, W)
    assert np.array_equal(r["Xq"], qx)
    assert np.array_equal(r["acc"], acc.astype(np.int32))
    assert np.array_equal(r["Y"].view(np.uint16), Yref.view(np.uint16))


def test_threshold_zero_is_fp_matmul_with_dequantized_weight():
    X, W, _ = workloads.make("tiny")
    X[:, 7] = 0.0  # an all-zero column is never an outlier, even at 0
    Wq, sW = oracle.quantize_weight(W)
    r = oracle.linear(X, Wq, sW, 0.0, stages=True)
    assert r["nO"] == X.shape[1] - 1 and 7 not in set(r["idx"])
    assert np.all(r["sX"] == 0) and np.all(r["Xq"] == 0)
    What = Wq.astype(np.float64) * sW.astype(np.float64)[:, None]
    ref = (X.astype(np.float64) @ What.T).astype(np.float16)
    assert ulp_distance(r["Y"], ref).max() <= 1


def test_error_bound_against_exact_matmul():
    """|Y - X W^T| within the closed-form quantization error bound.

    For normal columns x = sX*qx + ex, |ex| <= sX/2 and w = sW*qw + ew,
    |ew| <= sW/2, so |x w - sX sW qx qw| <= |x| sW/2 + |w| sX/2 + sX sW/4;
    outlier columns only carry the weight error |x| sW/2.  The fp32 products
    and the final fp16 rounding add at most a few ulps."""
    for name, thr in (("tiny", 6.0), ("tiny", np.inf), ("tiny", 0.0)):
        X, W, _ = workloads.make(name)
        Wq, sW = oracle.quantize_weight(W)
        r = oracle.linear(X, Wq, sW, thr, stages=True)
        x = X.astype(np.float64)
        w = W.astype(np.float64)
        exact = x @ w.T
        out = r["flags"].astype(bool)
        sX = r["sX"].astype(np.float64)
        sWd = sW.astype(np.float64)
        xn = np.abs(x[:, ~out])
        wn = np.abs(w[:, ~out])
        bound = (xn.sum(1)[:, None] * sWd[None, :] / 2
                 + sX[:, None] * wn.sum(1)[None, :] / 2
                 + (~out).sum() * sX[:, None] * sWd[None, :] / 4
                 + np.abs(x[:, out]).sum(1)[:, None] * sWd[None, :] / 2)
        y = r["Y"].astype(np.float64)
        slack = np.abs(y) * 2.0 ** -10 + 2.0 ** -24 + 1e-6 * bound
        assert np.all(np.abs(y - exact) <= bound + slack), name
        # and the decomposition is much better than the pure int8 path at 6.0
    X, W, _ = workloads.make("tiny")
    Wq, sW = oracle.quantize_weight(W)
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    e6 = np.abs(oracle.linear(X, Wq, sW, 6.0).astype(np.float64) - exact).mean()
    einf = np.abs(oracle.linear(X, Wq, sW, np.inf).astype(np.float64) - exact).mean()
    assert e6 < einf / 2


def test_joint_column_permutation():
    X, W, _ = workloads.make("tiny")
    Wq, sW = oracle.quantize_weight(W)
    r = oracle.linear(X, Wq, sW, 6.0, stages=True)
    perm = np.random.default_rng(5).permutation(X.shape[1])
    Xp = np.ascontiguousarray(X[:, perm])
    Wqp = np.ascontiguousarray(Wq[:, perm])
    rp = oracle.linear(Xp, Wqp, sW, 6.0, stages=True)
    assert np.array_equal(rp["Xq"], r["Xq"][:, perm])
    assert np.array_equal(rp["sX"], r["sX"])
    assert np.array_equal(rp["acc"], r["acc"])
    assert np.array_equal(np.sort(perm[rp["idx"]]), r["idx"])
    assert ulp_distance(rp["Y"], r["Y"]).max() <= 1


def test_linear_rows_matches_full_call():
    X, W, _ = workloads.make("tiny")
    Wq, sW = oracle.quantize_weight(W)
    full = oracle.linear(X, Wq, sW, 6.0, stages=True)
    rows = np.array([0, 3, 15])
    Y, idx, Xq, sX, acc = oracle.linear_rows(X, Wq, sW, 6.0, rows)
    assert np.array_equal(Y.view(np.uint16), full["Y"][rows].view(np.uint16))
    assert np.array_equal(idx, full["idx"]) and np.array_equal(acc, full["acc"][rows])


# --------------------------------------------------------------------------
# brute force (pure Python) on tiny shapes, special values included
# --------------------------------------------------------------------------

SPECIAL = [0.0, -0.0, 6.0, -6.0, 6.00390625, -6.00390625, 5.99609375, 1.0, -1.0,
           0.5, 127.0, 65504.0, -65504.0, 6.1e-05, 5.96e-08, 300.0, -3.5]


@st.composite
def _case(draw):
    T = draw(st.integers(1, 9))
    K = draw(st.integers(1, 17))
    N = draw(st.integers(1, 9))
    elem = st.one_of(st.sampled_from(SPECIAL),
                     st.floats(-8.0, 8.0, width=16),
                     st.floats(-200.0, 200.0, width=16))
    X = np.array(draw(st.lists(elem, min_size=T * K, max_size=T * K)), np.float16).reshape(T, K)
    W = np.array(draw(st.lists(st.floats(-2.0, 2.0, width=16), min_size=N * K,
                               max_size=N * K)), np.float16).reshape(N, K)
    if draw(st.booleans()):
        X[draw(st.integers(0, T - 1)), :] = 0.0  # an all-zero token
    thr = draw(st.sampled_from([6.0, 0.0, np.inf, 1.0, 100.0]))
    return X, W, thr


@settings(max_examples=150, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(_case())
def test_brute_force_agrees_bit_exactly(case):
    X, W, thr = case
    Wq, sW = oracle.quantize_weight(W)
    bWq, bsW = brute.quantize_weight(W.view(np.uint16).tolist())
    assert np.array_equal(Wq, np.array(bWq, np.int8).reshape(Wq.shape))
    assert np.array_equal(sW, np.array(bsW, np.float32))
    r = oracle.linear(X, Wq, sW, thr, stages=True)
    b = brute.linear(X.view(np.uint16).tolist(), bWq, bsW, thr)
    assert list(r["flags"]) == b["flags"]
    assert list(r["idx"]) == b["idx"]
    assert np.array_equal(r["Xq"], np.array(b["Xq"], np.int8).reshape(r["Xq"].shape))
    assert np.array_equal(r["sX"], np.array(b["sX"], np.float32))
    assert np.array_equal(r["acc"], np.array(b["acc"], np.int64).astype(np.int32))
    assert np.array_equal(r["Y"].view(np.uint16),
                          np.array(b["Y_bits"], np.uint16).reshape(r["Y"].shape))


def test_brute_force_on_tiny_workload_rows():
    X, W, _ = workloads.make("tiny")
    X = X[:4].copy()
    W = W[:24].copy()
    Wq, sW = oracle.quantize_weight(W)
    bWq, bsW = brute.quantize_weight(W.view(np.uint16).tolist())
    b = brute.linear(X.view(np.uint16).tolist(), bWq, bsW, 6.0)
    r = oracle.linear(X, Wq, sW, 6.0, stages=True)
    assert b["idx"] == list(r["idx"]) and len(b["idx"]) >= 1
    assert np.array_equal(r["Y"].view(np.uint16), np.array(b["Y_bits"], np.uint16))


# --------------------------------------------------------------------------
# fp16-weight variant: the outlier columns multiply the original fp16 weight
# (hncyxsy.com/news/230290, section 2.1: the weight sub-matrix of the outlier
# columns is extracted and multiplied in fp16)
# --------------------------------------------------------------------------

def _dyadic(rng, shape):
    """Values k/64 with |k| <= 256 (exact in fp16): every product is a
    multiple of 2^-12 below 16 in magnitude, so every fp64 sum of them here
    is exact whatever the order."""
    return (rng.integers(-256, 257, shape) / 64.0).astype(np.float16)


def test_fp16w_threshold_zero_is_the_rounded_exact_matmul():
    """At threshold 0 every column with a non-zero value is an outlier, the
    int8 part is 0, and Y must be the correctly rounded fp16 of X W^T."""
    rng = np.random.default_rng(3)
    X = _dyadic(rng, (12, 40))
    W = _dyadic(rng, (20, 40))
    X[:, 5] = 0.0   # all zero: not an outlier, and contributes nothing either way
    Wq, sW = oracle.quantize_weight(W)
    r = oracle.linear(X, Wq, sW, 0.0, stages=True, W16=W)
    assert np.all(r["Xq"] == 0) and 5 not in set(r["idx"])
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    assert np.array_equal(r["Y"].view(np.uint16), exact.astype(np.float16).view(np.uint16))


def test_fp16w_threshold_inf_equals_the_int8_path():
    X, W, _ = workloads.make("tiny")
    Wq, sW = oracle.quantize_weight(W)
    a = oracle.linear(X, Wq, sW, np.inf)
    b = oracle.linear(X, Wq, sW, np.inf, W16=W)
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16))


def test_fp16w_matches_dequantized_variant_on_grid_weights():
    """A weight already on its int8 grid with a power-of-two scale
    (W = q * 2^-e, some |q| = 127 per row) quantizes back to q and 2^-e
    exactly, so both variants multiply the outliers by the same values."""
    rng = np.random.default_rng(9)
    N, K = 24, 48
    q = rng.integers(-127, 128, (N, K))
    q[:, 0] = 127
    e = rng.integers(3, 9, N)
    W = (q * 2.0 ** -e[:, None]).astype(np.float16)
    Wq, sW = oracle.quantize_weight(W)
    assert np.array_equal(Wq, q.astype(np.int8)) and np.array_equal(sW, (2.0 ** -e).astype(np.float32))
    X, _, _ = workloads.make("tiny", T=10, K=K, N=N)
    for thr in (6.0, 0.0, 1.0):
        a = oracle.linear(X, Wq, sW, thr)
        b = oracle.linear(X, Wq, sW, thr, W16=W)
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), thr


def test_fp16w_error_bound_against_exact_matmul():
    """Only the normal columns carry quantization error now; the outlier
    columns are exact up to the fp64 sum."""
    for thr in (6.0, 0.0, np.inf):
        X, W, _ = workloads.make("tiny")
        Wq, sW = oracle.quantize_weight(W)
        r = oracle.linear(X, Wq, sW, thr, stages=True, W16=W)
        x = X.astype(np.float64)
        w = W.astype(np.float64)
        exact = x @ w.T
        out = r["flags"].astype(bool)
        sX = r["sX"].astype(np.float64)
        sWd = sW.astype(np.float64)
        bound = (np.abs(x[:, ~out]).sum(1)[:, None] * sWd[None, :] / 2
                 + sX[:, None] * np.abs(w[:, ~out]).sum(1)[None, :] / 2
                 + (~out).sum() * sX[:, None] * sWd[None, :] / 4)
        y = r["Y"].astype(np.float64)
        slack = np.abs(y) * 2.0 ** -10 + 2.0 ** -24 + 1e-6 * bound
        assert np.all(np.abs(y - exact) <= bound + slack), thr


@settings(max_examples=80, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(_case())
def test_fp16w_brute_force_agrees_bit_exactly(case):
    X, W, thr = case
    Wq, sW = oracle.quantize_weight(W)
    bWq, bsW = brute.quantize_weight(W.view(np.uint16).tolist())
    r = oracle.linear(X, Wq, sW, thr, W16=W)
    b = brute.linear(X.view(np.uint16).tolist(), bWq, bsW, thr, Wbits=W.view(np.uint16).tolist())
    assert np.array_equal(r.view(np.uint16), np.array(b["Y_bits"], np.uint16).reshape(r.shape))


# --------------------------------------------------------------------------
# SmoothQuant-style W8A8 (lowentro.cn notes, Q9-Q10; hncyxsy.com/news/230290,
# section 5.1): x.W^T = (x/s).(W*s)^T with per-channel factors, then absmax int8 on both sides
# --------------------------------------------------------------------------

def _sq_full(X, W, alpha, X_cal=None):
    X_cal = X if X_cal is None else X_cal
    s = oracle.sq_factors(oracle.column_absmax(X_cal), oracle.column_absmax(W), alpha)
    Wq, sW = oracle.sq_quantize_weight(W, s)
    r = oracle.sq_linear(X, s, Wq, sW, stages=True)
    r.update(s=s, Wq=Wq, sW=sW)
    return r


def test_sq_uniform_power_of_two_factor_is_the_plain_int8_path():
    """A factor 2^k shared by every channel scales X, W and both scales by
    exact powers of two: codes, accumulators and Y equal the plain
    vector-wise int8 product (itself pinned to numpy above)."""
    X, W, _ = workloads.make("tiny")
    Wq0, sW0 = oracle.quantize_weight(W)
    Y0 = oracle.linear(X, Wq0, sW0, np.inf)
    for k in (-3, 0, 5):
        s = np.full(X.shape[1], 2.0 ** k, np.float32)
        Wq, sW = oracle.sq_quantize_weight(W, s)
        assert np.array_equal(Wq, Wq0) and np.array_equal(sW, sW0 * np.float32(2.0 ** k))
        Y = oracle.sq_linear(X, s, Wq, sW)
        assert np.array_equal(Y.view(np.uint16), Y0.view(np.uint16)), k


def test_sq_factors_closed_forms():
    """alpha = 1 gives s = ax, alpha = 0 gives s = 1/aw, alpha = 0.5 gives
    sqrt(ax/aw); a channel whose activation or weight maximum is 0 keeps 1.
    (lowentro.cn notes, Q10: alpha = 1 moves all of the activation's range
    to the weight, alpha = 0 all of the weight's to the activation, 0.5
    splits it evenly.  The printed product form would give aw at alpha = 0,
    squaring the weight's range instead; the quotient is the reading that
    matches the answer's description, so that is what this pins.)"""
    ax = np.array([8.0, 0.5, 0.0, 3.0, 100.0], np.float32)
    aw = np.array([0.5, 2.0, 1.0, 0.0, 0.04], np.float32)
    live = (ax > 0) & (aw > 0)
    s1 = oracle.sq_factors(ax, aw, 1.0)
    assert np.array_equal(s1, np.where(live, ax, 1.0).astype(np.float32))
    s0 = oracle.sq_factors(ax, aw, 0.0)
    inv = 1.0 / np.where(live, aw.astype(np.float64), 1.0)
    assert np.array_equal(s0, np.where(live, inv, 1.0).astype(np.float32))
    s5 = oracle.sq_factors(ax, aw, 0.5)
    ref = np.sqrt(np.where(live, ax.astype(np.float64), 1.0) / np.where(live, aw.astype(np.float64), 1.0))
    assert np.all(ulp32(s5, np.where(live, ref, 1.0).astype(np.float32)) <= 1)


def ulp32(a, b):
    ia = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    ib = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def test_sq_half_migration_balances_channel_ranges():
    """With alpha = 0.5 and the call's own X as calibration, each channel's
    range becomes sqrt(ax * aw) on both sides."""
    X, W, _ = workloads.make("tiny")
    ax, aw = oracle.column_absmax(X), oracle.column_absmax(W)
    s = oracle.sq_factors(ax, aw, 0.5)
    xs = np.abs(X.astype(np.float32) * (np.float32(1.0) / s)).max(0)
    ws = np.abs(W.astype(np.float32) * s).max(0)
    target = np.sqrt(ax.astype(np.float64) * aw.astype(np.float64))
    ok = (ax > 0) & (aw > 0)
    assert np.allclose(xs[ok], target[ok], rtol=1e-6) and np.allclose(ws[ok], target[ok], rtol=1e-6)


def test_sq_error_bound_and_benefit():
    """|Y - X W^T| within the absmax bound of the smoothed operands, and
    smoothing beats the plain int8 product on channel outliers."""
    X, W, _ = workloads.make("tiny")
    r = _sq_full(X, W, 0.5)
    s = r["s"].astype(np.float64)
    xs = X.astype(np.float64) * (1.0 / s)
    ws = W.astype(np.float64) * s
    exact = X.astype(np.float64) @ W.astype(np.float64).T
    sX = r["sX"].astype(np.float64)
    sW = r["sW"].astype(np.float64)
    K = X.shape[1]
    bound = (np.abs(xs).sum(1)[:, None] * sW[None, :] / 2 + sX[:, None] * np.abs(ws).sum(1)[None, :] / 2
             + K * sX[:, None] * sW[None, :] / 4)
    y = r["Y"].astype(np.float64)
    assert np.all(np.abs(y - exact) <= bound * (1 + 1e-5) + np.abs(y) * 2.0 ** -10 + 2.0 ** -24)
    Wq0, sW0 = oracle.quantize_weight(W)
    plain = oracle.linear(X, Wq0, sW0, np.inf).astype(np.float64)
    assert np.abs(y - exact).mean() < 0.5 * np.abs(plain - exact).mean()


@settings(max_examples=60, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(_case(), st.sampled_from([0.0, 0.5, 0.8, 1.0]))
def test_sq_brute_force_agrees_bit_exactly(case, alpha):
    X, W, _ = case
    r = _sq_full(X, W, alpha)
    b = brute.sq_linear(X.view(np.uint16).tolist(), W.view(np.uint16).tolist(),
                        X.view(np.uint16).tolist(), alpha)
    assert np.array_equal(r["s"], np.array(b["s"], np.float32))
    assert np.array_equal(r["Wq"], np.array(b["Wq"], np.int8).reshape(r["Wq"].shape))
    assert np.array_equal(r["sW"], np.array(b["sW"], np.float32))
    assert np.array_equal(r["Xq"], np.array(b["Xq"], np.int8).reshape(r["Xq"].shape))
    assert np.array_equal(r["sX"], np.array(b["sX"], np.float32))
    assert np.array_equal(r["Y"].view(np.uint16), np.array(b["Y_bits"], np.uint16).reshape(r["Y"].shape))
