"""The handbook page's fp32 quantizer listing, restated (oracle; test infrastructure only).

Handbook page "端侧推理：llama.cpp 与 GGUF、MLX、ExecuTorch", section
"GGUF 的量化格式": a simplified PyTorch quantizer for Q8_0, Q4_0, Q4_1 and
Q4_K, applied to 4096*256 Student-t(5)*0.02 weights drawn after
``torch.manual_seed(0)``, followed by a printed table of bits/weight and
relative error ||deq - w|| / ||w||.

The listing keeps every scale in fp32 and never rounds it to fp16.  This
module restates that arithmetic in numpy (fp32, IEEE division, round half to
even, clamp after rounding) so the printed table can pin the semantics the
production quantizers in ``formats`` share with it (which element sets
Q4_0's signed scale, the min clamp of Q4_K, the 6-bit code ranges).  It is
not the production path: ``formats`` additionally stores scales as fp16.

Each function returns (dequantized fp32 weights, bits per weight) where the
bits per weight is the closed form the listing prints next to each format.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def _div(a, b):
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.divide(a, b, dtype=F32)


def q8_0(w):
    b = np.asarray(w, F32).reshape(-1, 32)
    d = _div(np.abs(b).max(axis=1, keepdims=True), F32(127))
    return (np.clip(np.rint(_div(b, d)), -127, 127) * d).reshape(-1), 8 + 16 / 32


def q4_0(w):
    b = np.asarray(w, F32).reshape(-1, 32)
    j = np.argmax(np.abs(b), axis=1)[:, None]
    d = _div(np.take_along_axis(b, j, axis=1), F32(-8))
    return (np.clip(np.rint(_div(b, d)), -8, 7) * d).reshape(-1), 4 + 16 / 32


def q4_1(w):
    b = np.asarray(w, F32).reshape(-1, 32)
    lo = b.min(axis=1, keepdims=True)
    hi = b.max(axis=1, keepdims=True)
    d = _div(hi - lo, F32(15))
    return (np.clip(np.rint(_div(b - lo, d)), 0, 15) * d + lo).reshape(-1), 4 + 32 / 32


def q4_k(w):
    b = np.asarray(w, F32).reshape(-1, 8, 32)
    lo = np.minimum(b.min(axis=2, keepdims=True), F32(0))
    hi = b.max(axis=2, keepdims=True)
    sc = _div(hi - lo, F32(15))
    mn = -lo
    dsc = _div(sc.max(axis=1, keepdims=True), F32(63))
    dmn = _div(mn.max(axis=1, keepdims=True), F32(63))
    sc_q = np.clip(np.rint(_div(sc, dsc)), 1, 63) * dsc
    mn_q = np.clip(np.rint(_div(mn, dmn)), 0, 63) * dmn
    q = np.clip(np.rint(_div(b + mn_q, sc_q)), 0, 15)
    return (q * sc_q - mn_q).reshape(-1), 4 + (6 + 6) * 8 / 256 + 2 * 16 / 256


LISTING = (("Q8_0", q8_0), ("Q4_0", q4_0), ("Q4_1", q4_1), ("Q4_K", q4_k))


def relative_error(deq, w) -> float:
    """||deq - w|| / ||w|| evaluated in float64."""
    w64 = np.asarray(w, np.float64)
    return float(np.linalg.norm(np.asarray(deq, np.float64) - w64) / np.linalg.norm(w64))


def page_weights() -> np.ndarray:
    """The listing's sample: torch.manual_seed(0), StudentT(5).sample((4096*256,)) * 0.02."""
    import torch  # CPU only: the page draws its sample with torch's generator

    torch.manual_seed(0)
    w = torch.distributions.StudentT(5.0).sample((4096 * 256,)) * 0.02
    return w.numpy().astype(F32)
