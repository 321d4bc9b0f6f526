"""HIP-graph capture of GEMV launches (how the bench and a decode step issue
them): every replay must equal the eager result bit for bit, with eager work
and synchronisations between replays."""
import numpy as np
import pytest

import block_quantized_decode_qgemv_amd as qg
import workloads
from oracle import formats as OF
from oracle import gemv as OG

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("fmt", ["q4_k", "q8_0", "q2_k"])
def test_graph_replays_match_eager(fmt):
    n, k, copies = 515, 4096, 3
    blks = [OF.quantize(fmt, workloads.student_t_weights(n, k, 4, c)) for c in range(copies)]
    w = [torch.from_numpy(OF.pack(fmt, b)).cuda() for b in blks]
    x = torch.from_numpy(workloads.normal((1, k), 4, 9)).cuda()
    ys = [torch.empty((1, n), device="cuda") for _ in range(copies)]
    eager = []
    for c in range(copies):
        qg.qgemv(fmt, w[c], x, ys[c], n, k, 1)
        torch.cuda.synchronize()
        eager.append(ys[c].clone())
        ok, ratio, _ = OG.check(ys[c].cpu().numpy(), OF.dequant(fmt, blks[c]), x.cpu().numpy())
        assert ok, ratio
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in range(copies):
            qg.qgemv(fmt, w[c], x, ys[c], n, k, 1, stream=stream)
    for rep in range(4):
        for yy in ys:
            yy.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for c in range(copies):
            assert torch.equal(ys[c].view(torch.int32), eager[c].view(torch.int32)), (rep, c)


def test_graph_capture_before_any_eager_call():
    """The first launch of a (format, batch) pair may sit inside a capture:
    the launcher's one-time occupancy query must not break the capture or
    change the kernel it picks (replays equal a later eager call)."""
    fmt, n, k, b = "q4_1", 6007, 2048, 6
    blk = OF.quantize(fmt, workloads.student_t_weights(n, k, 4, 21))
    w = torch.from_numpy(OF.pack(fmt, blk)).cuda()
    x = torch.from_numpy(workloads.normal((b, k), 4, 22)).cuda()
    y = torch.full((b, n), float("nan"), device="cuda")
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        qg.qgemv(fmt, w, x, y, n, k, b, stream=stream)
    y_eager = torch.empty_like(y)
    qg.qgemv(fmt, w, x, y_eager, n, k, b)
    torch.cuda.synchronize()
    ok, ratio, _ = OG.check(y_eager.cpu().numpy(), OF.dequant(fmt, blk), x.cpu().numpy())
    assert ok, ratio
    for rep in range(3):
        y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_eager.view(torch.int32)), rep
