"""The handbook page's weight sample (oracle; test infrastructure only).

Handbook page "端侧推理：llama.cpp 与 GGUF、MLX、ExecuTorch", section
"GGUF 的量化格式": the quantizer comparison draws 4096*256 Student-t(5)
weights scaled by 0.02 with torch's generator after seeding it with 0, and
prints each format's bits/weight and relative error for that sample.  Only
the draw lives here; the quantizers are those of ``formats`` (its
page-literal mode reproduces the printed table).
"""
from __future__ import annotations

import numpy as np


def page_weights() -> np.ndarray:
    """The page's sample as fp32: torch.manual_seed(0), then 4096*256 draws of
    StudentT(5) times 0.02, on the CPU."""
    import torch  # the page draws its sample with torch's CPU generator

    torch.manual_seed(0)
    w = torch.distributions.StudentT(5.0).sample((4096 * 256,)) * 0.02
    return w.numpy().astype(np.float32)
