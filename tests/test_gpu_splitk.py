"""GPU parity of the split-K GEMV (row-starved launches at batch 5 and up,
partial sums in the caller's workspace, fixed-order second pass) through the
C ABI: every format at 1024 x 4096 (64 row groups: split 4 ways on a
256-unit chip) and 4096 x 4096 (no split), batches 1, 3, 5 and 8, against
the oracle; results repeat bit for bit; with no workspace (or a short one)
the single-pass kernel runs and gives its own result."""
import numpy as np
import pytest

import block_quantized_decode_qgemv_amd as qg
import workloads
from oracle import formats as OF
from oracle import gemv as OG
from tests.test_gpu_gemv import dev, make_blocks

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def _call(fmt, w_d, x_d, n, k, b, ws=None, ws_bytes=0):
    y = torch.full((b, n), float("nan"), device="cuda")
    qg.qgemv(fmt, w_d, x_d, y, n, k, b, ws=ws, ws_bytes=ws_bytes)
    return y


@pytest.mark.parametrize("fmt", OF.FORMATS)
@pytest.mark.parametrize("n,k", [(1024, 4096), (4096, 4096), (1000, 8192)])
@pytest.mark.parametrize("b", [1, 3, 5, 8])
def test_splitk_parity_and_determinism(fmt, n, k, b):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    groups = -(-n // 16)
    want_split = 4 if groups * 4 <= cus else (2 if groups * 2 <= cus else 1)
    ws_bytes = qg.qgemv_workspace_size(fmt, n, k, b)
    assert ws_bytes == (want_split * b * n * 4 if b >= 5 and want_split > 1 else 0)
    blk = make_blocks(fmt, n, k, seed=51, tid=b)
    w_d = dev(OF.pack(fmt, blk))
    x = workloads.normal((b, k), 52, n + b)
    x_d = dev(x)
    ws = torch.full((max(ws_bytes, 16),), 0xFF, dtype=torch.uint8, device="cuda")  # NaN-filled partials
    y1 = _call(fmt, w_d, x_d, n, k, b, ws, ws_bytes)
    y2 = _call(fmt, w_d, x_d, n, k, b, ws, ws_bytes)
    torch.cuda.synchronize()
    ok, ratio, idx = OG.check(y1.cpu().numpy(), OF.dequant(fmt, blk), x)
    assert ok, f"{fmt} {n}x{k} B={b} split {want_split}: |err|/tol = {ratio:.3g} at {idx}"
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), "split-K results must repeat bit for bit"
    if ws_bytes:
        # no workspace, or one a float short: the single-pass kernel, within the bound too
        y_plain = _call(fmt, w_d, x_d, n, k, b)
        y_short = _call(fmt, w_d, x_d, n, k, b, ws, ws_bytes - 4)
        torch.cuda.synchronize()
        assert torch.equal(y_plain.view(torch.int32), y_short.view(torch.int32))
        ok, ratio, idx = OG.check(y_plain.cpu().numpy(), OF.dequant(fmt, blk), x)
        assert ok, ratio


def test_splitk_graph_replays_match_eager():
    fmt, n, k, b = "q4_k", 1024, 4096, 8
    blk = make_blocks(fmt, n, k, seed=53)
    w_d = dev(OF.pack(fmt, blk))
    x_d = dev(workloads.normal((b, k), 53, 1))
    ws_bytes = qg.qgemv_workspace_size(fmt, n, k, b)
    assert ws_bytes > 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    y = torch.empty((b, n), device="cuda")
    qg.qgemv(fmt, w_d, x_d, y, n, k, b, ws=ws, ws_bytes=ws_bytes)
    torch.cuda.synchronize()
    eager = y.clone()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        qg.qgemv(fmt, w_d, x_d, y, n, k, b, ws=ws, ws_bytes=ws_bytes, stream=stream)
    for _ in range(3):
        y.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), eager.view(torch.int32))
