"""Seeded synthetic inputs for the LLM.int8() mixed-precision linear.

This module only draws random numbers.  It holds none of the method's
arithmetic (no scales, no rounding to codes, no matmul), so that the CPU
oracle and the HIP path can both take their inputs from it without sharing
any computation.

The activations imitate what the pages describe for the hidden states of
7B-70B transformer layers: almost every value is small (N(0,1) here), a
handful of fixed feature dimensions carry values 20-100x larger on every
token (hncyxsy.com/news/230290, section 1; lowentro.cn "model quantization"
notes, Q4 and Q11), and the 13B shape adds token-wise outliers that hit
random positions (lowentro.cn notes, Q11).  Weights are N(0, std) like a
trained linear layer's.

Draw order for one configuration (``numpy.random.default_rng(seed)``):
  1. X  = standard_normal((T, K), float32)
  2. cols = sorted(choice(K, n_fixed, replace=False))
  3. X[:, cols] = sign * uniform(lo, hi), sign from choice([-1, 1]),
     drawn element-wise over all T rows
  4. (token-sparse configs) mask = random((T, K)) < rate outside cols;
     X[mask] = sign * uniform(sp_lo, sp_hi)
  5. (zero-outlier configs) skip 2-4 and redraw every |x| > 6 until none
     is left
  6. X -> float16
  7. W = standard_normal((N, K), float32) * std -> float16
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int            # tokens (rows of X, rows of Y)
    K: int            # hidden size (columns of X and of W)
    N: int            # output features (rows of W, columns of Y)
    n_fixed: int      # fixed outlier feature columns
    lo: float         # outlier magnitude range
    hi: float
    w_std: float
    sparse_rate: float = 0.0   # token-wise outlier rate (0 = none)
    sp_lo: float = 0.0
    sp_hi: float = 0.0
    no_outliers: bool = False  # redraw any |x| > 6
    threshold: float = 6.0
    seed: int = 0
    desc: str = ""

    @property
    def ops(self) -> int:
        """2*T*N*K, the operation count the effective-TOPS metric uses."""
        return 2 * self.T * self.N * self.K


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny", 16, 256, 256, 2, 20.0, 60.0, 0.02,
                 desc="tiny: X[16,256], 2 outlier columns ~U(20,60), W[256,256]"),
        Workload("decode_7b_attn", 8, 4096, 4096, 4, 20.0, 100.0, 0.02,
                 desc="decode-shaped 7B attention projection, T=8 K=4096 N=4096"),
        Workload("prefill_7b_ffn_up", 2048, 4096, 11008, 6, 20.0, 100.0, 0.02,
                 desc="prefill 7B FFN up-projection, T=2048 K=4096 N=11008"),
        Workload("prefill_7b_ffn_up_t4096", 4096, 4096, 11008, 6, 20.0, 100.0, 0.02,
                 desc="prefill 7B FFN up-projection, T=4096 K=4096 N=11008"),
        Workload("ffn_13b", 512, 5120, 13824, 8, 20.0, 100.0, 0.015,
                 sparse_rate=1e-4, sp_lo=7.0, sp_hi=30.0,
                 desc="13B FFN, T=512 K=5120 N=13824, fixed + token-sparse outliers"),
        Workload("ffn_70b_slice", 4096, 8192, 28672, 8, 20.0, 100.0, 0.01,
                 desc="70B-class FFN slice, T=4096 K=8192 N=28672"),
        Workload("ffn_70b_slice_no_outliers", 4096, 8192, 28672, 0, 0.0, 0.0, 0.01,
                 no_outliers=True,
                 desc="70B-class FFN slice with no outlier columns"),
        # Decode-time (few-token) FFN projections of the same model sizes:
        # up-projections have many output features, down-projections a
        # long K (the FFN width).  Same recipe as the attention projection.
        Workload("decode_7b_ffn_up", 8, 4096, 11008, 4, 20.0, 100.0, 0.02,
                 desc="decode-shaped 7B FFN up-projection, T=8 K=4096 N=11008"),
        Workload("decode_7b_ffn_down", 8, 11008, 4096, 4, 20.0, 100.0, 0.02,
                 desc="decode-shaped 7B FFN down-projection, T=8 K=11008 N=4096"),
        Workload("decode_13b_ffn_up", 16, 5120, 13824, 8, 20.0, 100.0, 0.015,
                 desc="decode-shaped 13B FFN up-projection, T=16 K=5120 N=13824"),
        Workload("decode_13b_ffn_down", 1, 13824, 5120, 8, 20.0, 100.0, 0.015,
                 desc="decode-shaped 13B FFN down-projection, one token, K=13824 N=5120"),
        Workload("decode_70b_ffn_down", 16, 28672, 8192, 8, 20.0, 100.0, 0.01,
                 desc="decode-shaped 70B FFN down-projection, T=16 K=28672 N=8192"),
    ]
}


def _signed_uniform(rng: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    sign = rng.choice(np.array([-1.0, 1.0], dtype=np.float32), size=shape)
    return (sign * rng.uniform(lo, hi, size=shape)).astype(np.float32)


def make_activation(w: Workload, seed: int | None = None,
                    T: int | None = None, K: int | None = None):
    """Return (X fp16 [T,K], fixed outlier columns) drawn per the module recipe."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    T = w.T if T is None else T
    K = w.K if K is None else K
    X = rng.standard_normal((T, K), dtype=np.float32)
    cols = np.zeros(0, dtype=np.int64)
    if w.no_outliers:
        bad = np.abs(X) > 6.0
        while bad.any():
            X[bad] = rng.standard_normal(int(bad.sum()), dtype=np.float32)
            bad = np.abs(X) > 6.0
    else:
        if w.n_fixed:
            cols = np.sort(rng.choice(K, w.n_fixed, replace=False)).astype(np.int64)
            X[:, cols] = _signed_uniform(rng, (T, len(cols)), w.lo, w.hi)
        if w.sparse_rate > 0.0:
            mask = rng.random((T, K)) < w.sparse_rate
            mask[:, cols] = False
            cnt = int(mask.sum())
            X[mask] = _signed_uniform(rng, (cnt,), w.sp_lo, w.sp_hi)
    return X.astype(np.float16), cols


def make_weight(w: Workload, seed: int | None = None,
                N: int | None = None, K: int | None = None) -> np.ndarray:
    """W fp16 [N,K] ~ N(0, std).  Drawn from its own stream (seed + 1)."""
    rng = np.random.default_rng((w.seed if seed is None else seed) + 1)
    N = w.N if N is None else N
    K = w.K if K is None else K
    W = rng.standard_normal((N, K), dtype=np.float32)
    W *= np.float32(w.w_std)
    return W.astype(np.float16)


def make(name: str, seed: int | None = None, **shape):
    """(X, W, fixed_cols) for a named workload; shape overrides T/K/N allowed."""
    w = WORKLOADS[name]
    if shape:
        w = dataclasses.replace(w, **shape)
    X, cols = make_activation(w, seed)
    W = make_weight(w, seed)
    return X, W, cols


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
