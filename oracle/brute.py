"""Pure-Python brute force of the LLM.int8() decomposition, for tiny shapes.

TEST INFRASTRUCTURE ONLY.  A second, independent implementation used to
cross-check oracle.c: Python floats (binary64) for arithmetic, ``struct``
for the rounding to binary32 ('f') and binary16 ('e'), Python's ``round``
(ties to even) for codes.  Nested loops, no numpy, so every step can be
read against the pages:

  scale = absmax / 127, q = round(r / scale) clipped to [-127, 127]
      (tqpw.cn/news/5683, section 2.1; lowentro.cn notes, Q2 and Q11);
  one scale per weight row and per activation row (hncyxsy.com/news/230290,
      section 2.1; notes Q3);
  columns with some |x| > threshold are outliers, multiplied in floating
      point and added to the dequantized int8 product (hncyxsy.com, 2.1;
      notes Q4).

fl32(a / b) and fl32(a * b) of binary32 operands equal the binary64 result
rounded to binary32 (binary64 carries more than 2*24 + 2 bits, so the double
rounding is innocuous); the helpers below rely on that.
"""
from __future__ import annotations

import math
import struct


def f32(x: float) -> float:
    """Round a Python float to the nearest binary32 (ties to even)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def h2f(bits: int) -> float:
    return struct.unpack("<e", struct.pack("<H", bits))[0]


def f2h(x: float) -> int:
    """Nearest binary16 bit pattern (ties to even); overflow -> +-inf."""
    try:
        return struct.unpack("<H", struct.pack("<e", x))[0]
    except OverflowError:
        return 0xFC00 if x < 0 else 0x7C00


def code(r: float, s: float) -> int:
    if s == 0.0:
        return 0
    q = round(f32(r / s))
    return max(-127, min(127, q))


def quantize_weight(Wbits):
    """Wbits: list of rows of binary16 bit patterns."""
    Wq, sW = [], []
    for row in Wbits:
        vals = [h2f(b) for b in row]
        s = f32(max([abs(v) for v in vals] + [0.0]) / 127.0)
        sW.append(s)
        Wq.append([code(v, s) for v in vals])
    return Wq, sW


def linear(Xbits, Wq, sW, threshold: float, Wbits=None):
    """Returns dict(flags, idx, Xq, sX, acc, Y_bits) for X given as bit rows.
    With Wbits (the fp16 weight as bit rows) the outlier columns are
    multiplied by the fp16 weight instead of the dequantized codes."""
    T = len(Xbits)
    K = len(Xbits[0]) if T else len(Wq[0]) if Wq else 0
    X = [[h2f(b) for b in row] for row in Xbits]
    flags = [0] * K
    for t in range(T):
        for j in range(K):
            if abs(X[t][j]) > threshold:
                flags[j] = 1
    idx = [j for j in range(K) if flags[j]]
    Xq, sX = [], []
    for t in range(T):
        normal = [abs(X[t][j]) for j in range(K) if not flags[j]]
        s = f32(max(normal + [0.0]) / 127.0)
        sX.append(s)
        Xq.append([0 if flags[j] else code(X[t][j], s) for j in range(K)])
    N = len(Wq)
    acc = [[sum(Xq[t][j] * Wq[n][j] for j in range(K)) for n in range(N)] for t in range(T)]
    Y = []
    for t in range(T):
        yrow = []
        for n in range(N):
            d = f32(f32(float(acc[t][n])) * sX[t])
            d = f32(d * sW[n])
            e = 0.0
            for j in idx:
                w = h2f(Wbits[n][j]) if Wbits is not None else float(Wq[n][j]) * sW[n]
                e += X[t][j] * w
            yrow.append(f2h(d + e))
        Y.append(yrow)
    return dict(flags=flags, idx=idx, Xq=Xq, sX=sX, acc=acc, Y_bits=Y)


def sq_linear(Xbits, Wbits, X_cal_bits, alpha: float):
    """SmoothQuant-style W8A8 (lowentro.cn notes, Q9-Q10; hncyxsy.com/news/230290,
    section 5.1), every step in Python: per-channel factors from the calibration rows and the
    weight, the smoothed weight and activation, absmax int8 on both, exact
    integer products.  Returns dict(s, Wq, sW, Xq, sX, acc, Y_bits)."""
    K = len(Wbits[0])
    ax = [max([abs(h2f(r[j])) for r in X_cal_bits] + [0.0]) for j in range(K)]
    aw = [max([abs(h2f(r[j])) for r in Wbits] + [0.0]) for j in range(K)]
    s = []
    for j in range(K):
        if ax[j] == 0.0 or aw[j] == 0.0:
            s.append(1.0)
        else:
            s.append(f32(math.pow(ax[j], alpha) / math.pow(aw[j], 1.0 - alpha)))
    Wq, sW = [], []
    for row in Wbits:
        ws = [f32(h2f(b) * s[j]) for j, b in enumerate(row)]
        sc = f32(max([abs(v) for v in ws] + [0.0]) / 127.0)
        sW.append(sc)
        Wq.append([code(v, sc) if sc > 0.0 else 0 for v in ws])
    Xq, sX = [], []
    for row in Xbits:
        xs = [f32(h2f(b) * f32(1.0 / s[j])) for j, b in enumerate(row)]
        sc = f32(max([abs(v) for v in xs] + [0.0]) / 127.0)
        sX.append(sc)
        Xq.append([code(v, sc) if sc > 0.0 else 0 for v in xs])
    acc = [[sum(a * b for a, b in zip(xr, wr)) for wr in Wq] for xr in Xq]
    Y = [[f2h(f32(f32(float(acc[t][n]) * sX[t]) * sW[n])) for n in range(len(Wq))]
         for t in range(len(Xq))]
    return dict(s=s, Wq=Wq, sW=sW, Xq=Xq, sX=sX, acc=acc, Y_bits=Y)
