"""Batch-1 (and batch-B) decode GEMV reference (oracle; test infrastructure only).

Handbook page "端侧推理：llama.cpp 与 GGUF、MLX、ExecuTorch", sections
"速度上限：带宽 ÷ 权重字节数" and the self-test answers: a single-user decode
step reads every weight once and forms, for each output, the dot product of
one quantized weight row with the activation vector, y = W x.  Batch B
stacks B activation rows: Y[b][n] = sum_k W[n][k] * X[b][k].

Reference arithmetic: the dequantized fp32 weights and fp32 activations are
widened to float64, where every fp32 x fp32 product is exact, and summed in
float64 (``gemv_ref``), or with ``math.fsum`` (``gemv_fsum``, exact up to one
final rounding; for tiny brute-force cases).

Acceptance bound: |y_gpu - y_ref| <= 2e-5 * sum_k |W[n][k] * X[b][k]| + 1e-7.
The relative part covers any fp32 summation order and the scale-hoisted form
S*sum(q*x) - Mn*sum(x) a kernel may use; the absolute part covers rows whose
terms cancel to ~0.

Parity: pinned by brute force (fsum) on tiny shapes and by integer-exact
cases (power-of-two scales, small integer activations), where any correct
summation order gives the exact value.
"""
from __future__ import annotations

import math

import numpy as np

REL_TOL = 2e-5
ABS_TOL = 1e-7


def gemv_ref(w_deq, x) -> np.ndarray:
    """float64 [B, N] = X[B, K] @ W[N, K]^T with exact products."""
    w64 = np.asarray(w_deq, np.float32).astype(np.float64)
    x64 = np.atleast_2d(np.asarray(x, np.float32)).astype(np.float64)
    return x64 @ w64.T


def gemv_bound(w_deq, x) -> np.ndarray:
    """float64 [B, N] = sum_k |W[n][k] * X[b][k]|."""
    w64 = np.abs(np.asarray(w_deq, np.float32).astype(np.float64))
    x64 = np.abs(np.atleast_2d(np.asarray(x, np.float32)).astype(np.float64))
    return x64 @ w64.T


def gemv_fsum(w_deq, x) -> np.ndarray:
    """Brute-force reference: one math.fsum per output (tiny shapes only)."""
    w = np.asarray(w_deq, np.float32)
    xs = np.atleast_2d(np.asarray(x, np.float32))
    out = np.empty((xs.shape[0], w.shape[0]), dtype=np.float64)
    for b in range(xs.shape[0]):
        for n in range(w.shape[0]):
            out[b, n] = math.fsum(float(w[n, k]) * float(xs[b, k]) for k in range(w.shape[1]))
    return out


def tolerance(w_deq, x) -> np.ndarray:
    return REL_TOL * gemv_bound(w_deq, x) + ABS_TOL


def check(y, w_deq, x):
    """Return (ok, worst ratio |err| / tol, index of the worst element)."""
    y = np.atleast_2d(np.asarray(y, np.float64))
    err = np.abs(y - gemv_ref(w_deq, x))
    tol = tolerance(w_deq, x)
    ratio = err / tol
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    return bool(np.all(err <= tol)), float(ratio[idx]), idx
