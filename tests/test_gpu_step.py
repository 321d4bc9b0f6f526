"""GPU parity of the decode step as the bench times it: a two-layer step
graph built by the bench's own StepChain (q/k/v 6144x4096, o 4096x4096,
gate/up 28672x4096, down 4096x14336, Q4_K, batch 1, each projection reading
the previous one's output), replayed several times with eager work between
replays.  After every replay, sampled rows of every launch's output are
checked against the oracle on that launch's actual input (the previous
launch's output, read back), and every replay equals the eager run bit for
bit.  Weights come from the C++ quantizer; the sampled rows' bytes are checked
against the oracle's quantizer first."""
import numpy as np
import pytest

import bench
import block_quantized_decode_qgemv_amd as qg
import workloads
from oracle import formats as OF
from oracle import gemv as OG
from oracle import norm as ON

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

SAMPLE = 24


def _layers(n_layers):
    """Per layer: packed device tensors, host fp32 sampled rows and their indices."""
    layers, host = [], []
    for li in range(n_layers):
        dev, rows_of = {}, {}
        for j, (name, n, k) in enumerate(bench.FUSED_LAYER):
            w = workloads.student_t_weights_device(n, k, 40 + li, j).cpu().numpy()
            packed = qg.qquant("q4_k", w, n_threads=16)
            rows = np.unique(np.concatenate([[0, 15, 16, n - 1], np.random.default_rng(li * 10 + j).integers(0, n, SAMPLE)]))
            sub = OF.quantize("q4_k", w[rows])
            _check_bytes(packed, sub, rows, n, k)
            dev[name] = torch.from_numpy(packed).to("cuda")
            rows_of[name] = (rows, OF.dequant("q4_k", sub))
            del w
        layers.append(dev)
        host.append(rows_of)
    return layers, host


def _check_bytes(packed, sub, rows, n, k):
    spec = OF.SPECS["q4_k"]
    cpr, mpr = (k // spec.block) * spec.code_bytes, (k // spec.block) * spec.meta_bytes
    cp = OF.codes_plane_size("q4_k", n, k)
    sp = OF.pack("q4_k", sub)
    scp = OF.codes_plane_size("q4_k", len(rows), k)
    np.testing.assert_array_equal(OF.deinterleave_rows(packed[:cp], n, cpr)[rows],
                                  OF.deinterleave_rows(sp[:scp], len(rows), cpr))
    np.testing.assert_array_equal(OF.deinterleave_rows(packed[cp:cp + n * mpr], n, mpr)[rows],
                                  OF.deinterleave_rows(sp[scp:scp + len(rows) * mpr], len(rows), mpr))


def _check_replay(chain, host, gammas, eps):
    for li, name, n, k, _, xin, y, norm in chain.records:
        rows, w_rows = host[li][name]
        x = xin.cpu().numpy().astype(np.float32)
        got = y.cpu().numpy()[0, rows]
        if norm:
            g = (np.ones(k, np.float32) if isinstance(gammas, str)
                 else gammas[li][0 if name == "qkv" else 1].cpu().numpy())
            ok, ratio, idx = ON.check(got[None], w_rows, x, g, eps)
        else:
            ok, ratio, idx = OG.check(got[None], w_rows, x)
        assert ok, f"layer {li} {name} ({n}x{k}): |err|/tol = {ratio:.3g} at sampled row {rows[idx[-1]]}"


@pytest.mark.parametrize("norms", [None, "vector", "unit"])
def test_two_layer_step_graph(norms):
    layers, host = _layers(2)
    stream = torch.cuda.Stream()
    x0 = torch.from_numpy(workloads.normal((1, 4096), 41, 1)).to("cuda")
    gammas = None
    if norms == "vector":
        gammas = [torch.from_numpy(1.0 + 0.25 * workloads.normal((2, 4096), 41, 2 + li)).float().to("cuda")
                  for li in range(2)]
    elif norms == "unit":
        gammas = "unit"
    eps = 1e-5
    chain = bench.StepChain(torch, qg, layers, x0, stream, gammas=gammas, eps=eps)
    assert len(chain.launches) == 8
    with torch.cuda.stream(stream):
        for fn in chain.launches:
            fn()
    torch.cuda.synchronize()
    _check_replay(chain, host, gammas, eps)
    eager = [rec[6].clone() for rec in chain.records]
    g = bench.capture(torch, stream, chain.launches)
    for rep in range(3):
        for rec in chain.records:
            rec[6].fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for rec, ref in zip(chain.records, eager):
            assert torch.equal(rec[6].view(torch.int32), ref.view(torch.int32)), (rep, rec[0], rec[1])
    _check_replay(chain, host, gammas, eps)
