"""HIP-graph capture of GEMV launches (how the bench and a decode step issue
them): every replay must equal the eager result bit for bit, with eager work
and synchronisations between replays."""
import numpy as np
import pytest

import block_quantized_decode_qgemv_amd as qg
import workloads
from oracle import formats as OF
from oracle import gemv as OG
from tests.test_gpu_gemv import make_blocks

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("fmt", ["q4_k", "q8_0", "q2_k", "tern3"])
def test_graph_replays_match_eager(fmt):
    n, k, copies = 515, 4096, 3
    blks = [make_blocks(fmt, n, k, seed=4, tid=c) for c in range(copies)]
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


def test_graph_norm_gemv_and_requant_replays():
    """A captured decode-layer fragment: the norm-fed GEMV (bin8 and Q4_K, two
    batch sizes) and a device re-quantization with its status word; every
    replay equals the eager results bit for bit, with eager work that
    overwrites the outputs, the workspace and the status in between."""
    n, k = 300, 2048
    g8 = np.random.default_rng(5)
    bits = workloads.binary_codes(n, k, 5, 1)
    sc = workloads.scale_bits_f16((n, k // 128), 5, 2)
    w8 = torch.from_numpy(OF.pack("bin8", OF.bin8_from_codes(bits, sc))).cuda()
    blk = OF.quantize("q4_k", workloads.student_t_weights(n, k, 5, 3))
    wk = torch.from_numpy(OF.pack("q4_k", blk)).cuda()
    x = torch.from_numpy((workloads.normal((3, k), 5, 4) * 6).astype(np.float32)).cuda()
    gamma = torch.from_numpy((1 + 0.25 * g8.standard_normal(k)).astype(np.float32)).cuda()
    ya, yb = torch.empty((1, n), device="cuda"), torch.empty((3, n), device="cuda")
    q2 = torch.empty(qg.qg_packed_size("q2_k", n, k), dtype=torch.uint8, device="cuda")
    ws_bytes = qg.qrequant_workspace_size(n, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    status = torch.empty(1, dtype=torch.int32, device="cuda")

    def fragment(stream=None):
        qg.qgemv_rmsnorm("bin8", w8, x[:1], gamma, 1e-5, ya, n, k, 1, stream=stream)
        qg.qgemv_rmsnorm("q4_k", wk, x, gamma, 1e-5, yb, n, k, 3, stream=stream)
        qg.qrequant("q4_k", wk, "q2_k", q2, n, k, ws, ws_bytes, status, stream=stream)

    fragment()
    torch.cuda.synchronize()
    eager = [ya.clone(), yb.clone(), q2.clone()]
    assert int(status.item()) == 0
    np.testing.assert_array_equal(eager[2].cpu().numpy(),
                                  OF.pack("q2_k", OF.quantize("q2_k", OF.dequant("q4_k", blk))))
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fragment(stream)
    for rep in range(4):
        ya.fill_(float("nan"))
        yb.fill_(float("nan"))
        q2.fill_(0x5A)
        ws.fill_(0xAB)
        status.fill_(-99)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, rep
        for got, want in zip((ya, yb, q2), eager):
            assert torch.equal(got, want), rep
