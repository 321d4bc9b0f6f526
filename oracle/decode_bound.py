"""Decode speed bound (oracle; test infrastructure only).

Handbook page "端侧推理：llama.cpp 与 GGUF、MLX、ExecuTorch", section
"速度上限：带宽 ÷ 权重字节数", its printed device table and its exercise: at
batch 1 every decode step reads all weights once, so

    tokens/s <= effective bandwidth / quantized weight bytes,

with the page taking the effective bandwidth as 70 % of the nominal figure.
Parity: pinned by the page's printed device table and exercise answers.
"""
from __future__ import annotations


def tokens_per_s(bandwidth_bytes_per_s: float, weight_bytes: float, efficiency: float = 0.7) -> float:
    return bandwidth_bytes_per_s * efficiency / weight_bytes


def max_weight_bytes(bandwidth_bytes_per_s: float, tokens_per_second: float, efficiency: float = 0.7) -> float:
    return bandwidth_bytes_per_s * efficiency / tokens_per_second


def model_bytes(n_params: float, bits_per_weight: float) -> float:
    return n_params * bits_per_weight / 8.0
