"""Routed MoE expert layer at decode (oracle; test infrastructure only).

Sources:
* Flash-MoE page ("Flash-MoE：在笔记本上运行 397B 参数大模型"), sections
  "模型架构" (512 experts per layer, K=4 active plus one shared expert,
  hidden 4096), "Metal 计算着色器" (fused SwiGLU; fused MoE combine +
  residual + sigmoid gate) and "每层流水线" (softmax + top-K routing).
* EPM README, section "正確性": an expert's forward checked against a NumPy
  recompute, the routed matmul (llama.cpp ``mul_mat_id``) as the semantics,
  and stage-wise teacher forcing (feeding one side's SwiGLU intermediate to
  the other) to localise differences.

Per token t (float64 throughout):
    p      = softmax(logits_t)                     (max-subtracted)
    e_1..K = the K largest p, descending; ties go to the lower expert index
    w_k    = p[e_k]                                (no renormalisation unless asked)
    for e in {e_1..e_K, shared}:
        g = W_gate,e x_t ; u = W_up,e x_t ; h = silu(g) * u ; o_e = W_down,e h
        with silu(z) = z / (1 + exp(-z))
    out_t  = residual_t + sum_k w_k o_{e_k} + sigmoid(s_t) o_shared

Readings (pages silent): the sigmoid gate multiplies the shared expert's
output and its logit s_t is a per-token input; the shared expert has the
routed experts' intermediate width; the residual is a separate input; the
top-K weights are not renormalised (renormalisation is an option); no norm.

Parity: pinned by special cases that reduce to closed forms -- identical
experts (out = residual + (sum_k w_k + sigmoid(s)) E(x)), a shared logit of
-inf removing the shared path, a dominant logit fixing the route -- and by a
brute-force top-K over all subsets on small E.
"""
from __future__ import annotations

import math

import numpy as np

from . import gemv as _gemv


def softmax64(logits) -> np.ndarray:
    """Softmax over the last axis in float64, max-subtracted.  A NaN logit
    counts as -inf (the pages do not say; this is the stated reading)."""
    z = np.asarray(logits, np.float32).astype(np.float64)
    z = np.where(np.isnan(z), -np.inf, z)
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


def route(logits, top_k: int, renorm: bool = False):
    """Return (ids [T, K] int64, weights [T, K] float64, p [T, E] float64)."""
    p = softmax64(logits)
    t, e = p.shape
    ids = np.empty((t, top_k), dtype=np.int64)
    for i in range(t):
        # descending p; equal p keeps the lower index first (stable sort on -p)
        order = np.argsort(-p[i], kind="stable")
        ids[i] = order[:top_k]
    w = np.take_along_axis(p, ids, axis=1)
    if renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return ids, w, p


def route_margin(logits, top_k: int) -> np.ndarray:
    """Relative gap between the K-th and (K+1)-th probability, per token."""
    p = np.sort(softmax64(logits), axis=-1)[:, ::-1]
    return (p[:, top_k - 1] - p[:, top_k]) / p[:, top_k - 1]


def silu(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(-z))


def sigmoid(z):
    z = np.asarray(z, np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def _rows(x) -> np.ndarray:
    """Activation rows as float64 [B, H]: fp32 inputs widened exactly, float64
    inputs (an activation the oracle itself computed, such as a normalised x)
    taken as they are, without rounding to fp32."""
    a = np.atleast_2d(np.asarray(x))
    if a.dtype != np.float64:
        a = a.astype(np.float32)
    return a.astype(np.float64)


def _gemv64(w, x) -> np.ndarray:
    """W x over the rows of x, exact products, float64 sums."""
    return _rows(x) @ np.asarray(w, np.float32).astype(np.float64).T


def expert_forward(wg, wu, wd, x):
    """One expert on activation rows x [B, H]: returns (g, u, h, o), float64."""
    g = _gemv64(wg, x)
    u = _gemv64(wu, x)
    h = silu(g) * u
    o = np.asarray(h, np.float64) @ np.asarray(wd, np.float32).astype(np.float64).T
    return g, u, h, o


def moe_ref(w_gate, w_up, w_down, x, residual, logits, shared_logit, top_k: int, renorm: bool = False):
    """Full layer.  w_gate/w_up: [E+1] of [I, H]; w_down: [E+1] of [H, I]
    (expert E is the shared one); x, residual: [T, H]; logits: [T, E];
    shared_logit: [T].  Returns a dict with out [T, H] and the intermediates."""
    x = _rows(x)
    t = x.shape[0]
    e = len(w_gate) - 1
    ids, w, _ = route(logits, top_k, renorm)
    sig = sigmoid(np.asarray(shared_logit, np.float32))
    out = np.asarray(residual, np.float32).astype(np.float64).copy()
    h_all = np.empty((t, top_k + 1, np.asarray(w_gate[0]).shape[0]))
    o_all = np.empty((t, top_k + 1, x.shape[1]))
    for i in range(t):
        slots = list(ids[i]) + [e]
        for k, ex in enumerate(slots):
            _, _, h, o = expert_forward(w_gate[ex], w_up[ex], w_down[ex], x[i:i + 1])
            h_all[i, k] = h[0]
            o_all[i, k] = o[0]
        for k in range(top_k):
            out[i] += w[i, k] * o_all[i, k]
        out[i] += sig[i] * o_all[i, top_k]
    return {"out": out, "ids": ids, "weights": w, "sigma": sig, "h": h_all, "o": o_all}


# ----------------------------------------------------------------------------
# Tolerances propagated stage by stage from the GEMV bound.

COMBINE_REL = 2e-6   # fp32 softmax over E terms, sigmoid, and the 6-term combine
ACT_REL = 1e-6       # fp32 silu(g) * u beyond the propagated GEMV errors


def h_tolerance(wg, wu, x, rel: float = _gemv.REL_TOL):
    """Bound on |h_gpu - h_ref| for one expert and activation rows x, the
    gate/up GEMVs within rel * sum |w x| + ABS_TOL."""
    g = _gemv64(wg, x)
    u = _gemv64(wu, x)
    ax = np.abs(_rows(x))
    dg = rel * (ax @ np.abs(np.asarray(wg, np.float32).astype(np.float64)).T) + _gemv.ABS_TOL
    du = rel * (ax @ np.abs(np.asarray(wu, np.float32).astype(np.float64)).T) + _gemv.ABS_TOL
    s = sigmoid(g)
    dsilu = s * (1.0 + g * (1.0 - s))
    h = silu(g) * u
    return np.abs(dsilu * u) * dg + np.abs(silu(g)) * du + dg * du + ACT_REL * np.abs(h)


def o_tolerance(wd, h, dh):
    """Bound on |o_gpu - o_ref| given the reference h and its bound dh."""
    wd64 = np.abs(np.asarray(wd, np.float32).astype(np.float64))
    h = np.atleast_2d(h)
    dh = np.atleast_2d(dh)
    return _gemv.REL_TOL * (np.abs(h) @ wd64.T) + dh @ wd64.T + _gemv.ABS_TOL


def out_tolerance(w_gate, w_up, w_down, x, residual, ref, rel: float = _gemv.REL_TOL) -> np.ndarray:
    """Bound on |out_gpu - out_ref|; rel is the gate/up GEMV bound's relative part."""
    x = _rows(x)
    t = x.shape[0]
    top_k = ref["ids"].shape[1]
    e = len(w_gate) - 1
    tol = np.empty_like(ref["out"])
    for i in range(t):
        slots = list(ref["ids"][i]) + [e]
        coef = list(ref["weights"][i]) + [float(ref["sigma"][i])]
        acc = np.zeros(x.shape[1])
        mag = np.abs(np.asarray(residual, np.float32)[i].astype(np.float64))
        for k, ex in enumerate(slots):
            dh = h_tolerance(w_gate[ex], w_up[ex], x[i:i + 1], rel)
            do = o_tolerance(w_down[ex], ref["h"][i, k][None], dh)[0]
            acc += coef[k] * do
            mag += coef[k] * np.abs(ref["o"][i, k])
        tol[i] = acc + COMBINE_REL * mag
    return tol


def interleave_gate_up(wg, wu) -> np.ndarray:
    """[2I, H] with row 2i = gate row i and row 2i+1 = up row i."""
    wg = np.asarray(wg)
    out = np.empty((2 * wg.shape[0], wg.shape[1]), dtype=wg.dtype)
    out[0::2] = wg
    out[1::2] = wu
    return out


def top_k_bruteforce(p_row, top_k: int):
    """Best K-subset by total probability, ties to the lexicographically
    smallest index set (for pins on small E)."""
    import itertools

    best = None
    for comb in itertools.combinations(range(len(p_row)), top_k):
        key = (-math.fsum(p_row[list(comb)]), comb)
        if best is None or key < best:
            best = key
    return sorted(best[1], key=lambda j: (-p_row[j], j))
