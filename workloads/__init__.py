"""Seeded synthetic inputs shared by the oracle, the tests and the bench.

This module only draws random numbers.  It holds none of the quantizers',
the GEMV's or the MoE layer's arithmetic, so the oracle and the HIP path can
both take their inputs from here without sharing any of the method.

Recipes (shapes and distributions follow the pages' workloads):

* weights: Student-t with 5 degrees of freedom times 0.02, the heavy-tailed
  distribution of the quantizer comparison on the handbook page (edge
  inference chapter, section on GGUF quantization formats).  Drawn in float64
  by numpy and rounded once to float32.
* activations, router logits, shared-gate logits, residuals: N(0, 1) float32.
* ternary codes: i.i.d. {-1, 0, +1} with probability 1/3 each; 1-bit codes:
  i.i.d. {0, 1} with probability 1/2.  Their per-128 scales are fp16 bit
  patterns drawn uniformly from [0x211F, 0x27AE], i.e. values in roughly
  [0.01, 0.03], the magnitude of a 0.02-scale weight.

Every generator takes an explicit integer seed and a tensor id, and builds its
stream as ``numpy.random.default_rng(SeedSequence([seed, tensor_id]))``, so a
tensor is reproducible on its own without drawing all tensors before it.

The ``*_device`` generators draw the same distributions with torch's device
generator (seeded from seed and tensor id), for the bench's multi-gigabyte
inputs: numpy needs about 120 ns per Student-t sample on the host.  Student-t
is drawn as Z / sqrt(V / 5) with Z ~ N(0, 1) and V = 2 Gamma(5/2) ~ chi^2(5).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rng_for",
    "student_t_weights",
    "normal",
    "ternary_codes",
    "binary_codes",
    "scale_bits_f16",
    "single_q4k_case",
    "student_t_weights_device",
    "normal_device",
]

STUDENT_T_DOF = 5.0
STUDENT_T_SCALE = 0.02
# fp16 bit patterns bracketing ~0.01 .. ~0.03 (both ends are normal fp16 values).
SCALE_BITS_LO = 0x211F
SCALE_BITS_HI = 0x27AE


def rng_for(seed: int, tensor_id: int) -> np.random.Generator:
    """Independent stream for tensor ``tensor_id`` under run seed ``seed``."""
    return np.random.default_rng(np.random.SeedSequence([int(seed), int(tensor_id)]))


def student_t_weights(n: int, k: int, seed: int = 0, tensor_id: int = 0) -> np.ndarray:
    """float32 [n, k] weights, Student-t(5) * 0.02."""
    g = rng_for(seed, tensor_id)
    return (g.standard_t(STUDENT_T_DOF, size=(n, k)) * STUDENT_T_SCALE).astype(np.float32)


def normal(shape, seed: int = 0, tensor_id: int = 0) -> np.ndarray:
    """float32 N(0, 1) array of the given shape."""
    g = rng_for(seed, tensor_id)
    return g.standard_normal(size=shape).astype(np.float32)


def ternary_codes(n: int, k: int, seed: int = 0, tensor_id: int = 0) -> np.ndarray:
    """int8 [n, k] codes in {-1, 0, +1}, each with probability 1/3."""
    g = rng_for(seed, tensor_id)
    return (g.integers(0, 3, size=(n, k), dtype=np.int8) - 1).astype(np.int8)


def binary_codes(n: int, k: int, seed: int = 0, tensor_id: int = 0) -> np.ndarray:
    """uint8 [n, k] codes in {0, 1}, each with probability 1/2."""
    g = rng_for(seed, tensor_id)
    return g.integers(0, 2, size=(n, k), dtype=np.uint8)


def scale_bits_f16(shape, seed: int = 0, tensor_id: int = 0) -> np.ndarray:
    """uint16 fp16 bit patterns, uniform over [SCALE_BITS_LO, SCALE_BITS_HI]."""
    g = rng_for(seed, tensor_id)
    return g.integers(SCALE_BITS_LO, SCALE_BITS_HI + 1, size=shape, dtype=np.uint16)


def single_q4k_case(n: int = 1024, k: int = 1024, seed: int = 0):
    """The single-GEMV case: one ``default_rng(seed)`` draws W first, then x.

    Returns (W float32 [n, k], x float32 [1, k]).
    """
    g = np.random.default_rng(seed)
    w = (g.standard_t(STUDENT_T_DOF, size=(n, k)) * STUDENT_T_SCALE).astype(np.float32)
    x = g.standard_normal(size=(1, k)).astype(np.float32)
    return w, x


def _device_generator(seed: int, tensor_id: int, device):
    import torch

    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(tensor_id)) % (1 << 62))
    return g


def student_t_weights_device(n: int, k: int, seed: int = 0, tensor_id: int = 0, device="cuda"):
    """float32 [n, k] torch tensor on ``device``, Student-t(5) * 0.02."""
    import torch

    g = _device_generator(seed, tensor_id, device)
    z = torch.randn((n, k), generator=g, device=device, dtype=torch.float32)
    v = torch._standard_gamma(torch.full((n, k), STUDENT_T_DOF / 2, device=device, dtype=torch.float32),
                              generator=g) * 2.0
    return z * torch.rsqrt(v / STUDENT_T_DOF) * STUDENT_T_SCALE


def normal_device(shape, seed: int = 0, tensor_id: int = 0, device="cuda"):
    """float32 N(0, 1) torch tensor on ``device``."""
    import torch

    return torch.randn(shape, generator=_device_generator(seed, tensor_id, device), device=device,
                       dtype=torch.float32)
