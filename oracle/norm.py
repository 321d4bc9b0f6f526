"""RMS normalisation feeding a quantized projection (oracle; test
infrastructure only).

Flash-MoE page ("Flash-MoE：在笔记本上运行 397B 参数大模型"):
* section "Metal 计算着色器" lists RMS normalisation as a GPU kernel done in
  two passes -- a reduction of the sum of squares, then its application;
* section "延迟 GPU 专家计算" keeps the combine + residual + norm on the GPU,
  where it feeds the next layer's projection directly.

Readings (the pages name the norm but print no formula): the standard RMS
norm with a learned per-channel gain gamma and a stabiliser eps added under
the square root,

    rms(x)    = sqrt( (1/K) sum_k x_k^2 + eps )            (pass 1)
    xhat_k    = x_k * gamma_k / rms(x)                      (pass 2)

and the projection that consumes it is the decode GEMV, y = W xhat, so the
fused call computes Y[b][n] = sum_k W[n][k] xhat[b][k].  Each batch row is
normalised on its own.

Reference arithmetic: float64 throughout (fp32 inputs widened; xhat is kept
in float64, never rounded to fp32).

Acceptance bound: |y - y_ref| <= 3e-5 * sum_k |W[n][k] xhat[b][k]| + 1e-7.
Of the relative part, 2e-5 is the plain GEMV's bound applied to xhat and the
rest covers the fp32 sum of squares (a sum of K positive terms, whose
relative error is at most its longest sequential chain times the unit
roundoff, halved by the square root) and the fp32 square root and products.

The MoE layer fed through the same norm (every expert sees xhat; the
residual is the caller's, the un-normalised x in a pre-norm block) is the
moe oracle applied to the float64 xhat, with the gate/up GEMV bound widened
to this module's.

Parity: pinned by hand-computed vectors, closed forms (constant x gives the
row sums of W; a zero vector gives zero with eps > 0), the invariants of the
definition (scale invariance with eps = 0; unit mean square of xhat with
gamma = 1, eps = 0), and the identity y * rms(x) = W (gamma * x) against the
separately pinned GEMV oracle.
"""
from __future__ import annotations

import numpy as np

from . import moe as _moe

REL_TOL = 3e-5
ABS_TOL = 1e-7


def rms(x, eps: float) -> np.ndarray:
    """Pass 1: float64 [B] = sqrt(mean_k x[b][k]^2 + eps)."""
    x64 = np.atleast_2d(np.asarray(x, np.float32)).astype(np.float64)
    return np.sqrt(np.mean(x64 * x64, axis=1) + float(np.float32(eps)))


def rmsnorm_ref(x, gamma, eps: float) -> np.ndarray:
    """Pass 2: float64 [B, K] = x * gamma / rms(x), row by row."""
    x64 = np.atleast_2d(np.asarray(x, np.float32)).astype(np.float64)
    g64 = np.asarray(gamma, np.float32).astype(np.float64)
    return x64 * g64[None, :] / rms(x, eps)[:, None]


def gemv_rmsnorm_ref(w_deq, x, gamma, eps: float) -> np.ndarray:
    """float64 [B, N] = W rmsnorm(x), each row of x normalised on its own."""
    w64 = np.asarray(w_deq, np.float32).astype(np.float64)
    return rmsnorm_ref(x, gamma, eps) @ w64.T


def tolerance(w_deq, x, gamma, eps: float) -> np.ndarray:
    w64 = np.abs(np.asarray(w_deq, np.float32).astype(np.float64))
    return REL_TOL * (np.abs(rmsnorm_ref(x, gamma, eps)) @ w64.T) + ABS_TOL


def check(y, w_deq, x, gamma, eps: float):
    """Return (ok, worst ratio |err| / tol, index of the worst element)."""
    y = np.atleast_2d(np.asarray(y, np.float64))
    err = np.abs(y - gemv_rmsnorm_ref(w_deq, x, gamma, eps))
    tol = tolerance(w_deq, x, gamma, eps)
    ratio = err / tol
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    return bool(np.all(err <= tol)), float(ratio[idx]), idx



def moe_rmsnorm_ref(w_gate, w_up, w_down, x, gamma, eps: float, residual, logits, shared_logit, top_k: int,
                    renorm: bool = False):
    """The routed expert layer on rmsnorm(x) (see oracle.moe.moe_ref)."""
    return _moe.moe_ref(w_gate, w_up, w_down, rmsnorm_ref(x, gamma, eps), residual, logits, shared_logit,
                        top_k, renorm)


def moe_rmsnorm_tolerance(w_gate, w_up, w_down, x, gamma, eps: float, residual, ref) -> np.ndarray:
    return _moe.out_tolerance(w_gate, w_up, w_down, rmsnorm_ref(x, gamma, eps), residual, ref, rel=REL_TOL)
