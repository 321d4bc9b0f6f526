"""GPU parity of the RMS-normalising GEMV (qgemv_rmsnorm) against the oracle,
through the C ABI: every format, batches 1..8, ragged row groups, K tails of
the 32-weight formats, the widest workgroup, the eps edge cases, and the
decode layer's full projection shapes on sampled rows."""
import numpy as np
import pytest

import block_quantized_decode_qgemv_amd as qg
import workloads
from oracle import formats as OF
from oracle import norm as ON

from .test_gpu_gemv import check_sampled_bytes, dev, full_weights, make_blocks, sampled_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def residual_stream(b, k, seed, tid):
    """Activations entering a norm: a residual stream well away from unit RMS."""
    return (workloads.normal((b, k), seed, tid) * np.float32(6.0)).astype(np.float32)


def gain(k, seed, tid):
    return (1.0 + 0.25 * workloads.normal((1, k), seed, tid)[0]).astype(np.float32)


def run_norm(fmt, packed, x, gamma, eps, n, k):
    b = x.shape[0]
    y_d = torch.full((b, n), float("nan"), device="cuda")
    qg.qgemv_rmsnorm(fmt, dev(packed), dev(x), None if gamma is None else dev(gamma), eps, y_d, n, k, b)
    torch.cuda.synchronize()
    return y_d.cpu().numpy()


def assert_norm_parity(y, w_deq, x, gamma, eps, label):
    ok, ratio, idx = ON.check(y, w_deq, x, gamma, eps)
    assert ok, f"{label}: worst |err|/tol = {ratio:.3g} at {idx}"


SHAPES = [(1, 1), (67, 4), (130, 16), (9, 56)]  # (N, K in blocks of 256)


@pytest.mark.parametrize("fmt", OF.FORMATS)
@pytest.mark.parametrize("b", [1, 2, 3, 8])
@pytest.mark.parametrize("n,kb", SHAPES)
def test_rmsnorm_gemv_parity(fmt, b, n, kb):
    k = 256 * kb
    blk = make_blocks(fmt, n, k, seed=21, tid=5 * n + kb)
    x, g = residual_stream(b, k, 21, 400 + b), gain(k, 21, 500 + kb)
    y = run_norm(fmt, OF.pack(fmt, blk), x, g, 1e-6, n, k)
    assert_norm_parity(y, OF.dequant(fmt, blk), x, g, 1e-6, f"{fmt} B={b} N={n} K={k}")


@pytest.mark.parametrize("fmt", ["q4_k", "q4_1", "q2_k", "bin8"])
@pytest.mark.parametrize("b", [4, 5, 6, 7])
def test_rmsnorm_gemv_mid_batches(fmt, b):
    """Batches 4 to 7 (four-row blocks, one wide block, the unclamped loop)."""
    n, k = 45, 2048
    blk = make_blocks(fmt, n, k, seed=29, tid=b)
    x, g = residual_stream(b, k, 29, b), gain(k, 29, 1)
    y = run_norm(fmt, OF.pack(fmt, blk), x, g, 1e-6, n, k)
    assert_norm_parity(y, OF.dequant(fmt, blk), x, g, 1e-6, f"{fmt} B={b}")


@pytest.mark.parametrize("fmt", OF.FORMATS)
@pytest.mark.parametrize("b", [1, 5, 8])
def test_rmsnorm_gemv_widest_workgroup(fmt, b):
    """K = 16384: the widest workgroup and, at larger batches, several K
    slices whose sums of squares are combined across waves."""
    n, k = 33, 16384
    blk = make_blocks(fmt, n, k, seed=22, tid=b)
    x, g = residual_stream(b, k, 22, b), gain(k, 22, 99)
    y = run_norm(fmt, OF.pack(fmt, blk), x, g, 1e-5, n, k)
    assert_norm_parity(y, OF.dequant(fmt, blk), x, g, 1e-5, f"{fmt} B={b} N={n} K={k}")


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "q4_1"])
@pytest.mark.parametrize("k", [32, 160, 4064])
def test_rmsnorm_gemv_short_blocks(fmt, k):
    """32-weight formats at K off the 256 grid: the sum of squares must cover
    the ragged tail once, like the dot products."""
    n = 37
    blk = make_blocks(fmt, n, k, seed=23, tid=k)
    x, g = residual_stream(3, k, 23, k), gain(k, 23, k + 1)
    y = run_norm(fmt, OF.pack(fmt, blk), x, g, 1e-6, n, k)
    assert_norm_parity(y, OF.dequant(fmt, blk), x, g, 1e-6, f"{fmt} N={n} K={k}")


@pytest.mark.parametrize("fmt", ["q4_k", "q8_0"])
def test_rmsnorm_gemv_eps_cases(fmt):
    """eps = 0 on nonzero rows; a zero row with eps > 0 gives exactly zero;
    a tiny-RMS row where eps dominates; a zero row with eps = 0 is 0/0."""
    n, k = 20, 1024
    blk = make_blocks(fmt, n, k, seed=24)
    packed, w_deq = OF.pack(fmt, blk), OF.dequant(fmt, blk)
    g = gain(k, 24, 1)
    x = residual_stream(3, k, 24, 2)
    x[1] = 0.0
    x[2] *= np.float32(1e-4)
    y = run_norm(fmt, packed, x, g, 0.5, n, k)
    assert_norm_parity(y, w_deq, x, g, 0.5, f"{fmt} eps=0.5")
    assert np.all(y[1] == 0.0)
    y0 = run_norm(fmt, packed, x[[0, 2]], g, 0.0, n, k)
    assert_norm_parity(y0, w_deq, x[[0, 2]], g, 0.0, f"{fmt} eps=0")
    yz = run_norm(fmt, packed, x[[1]], g, 0.0, n, k)
    assert np.all(np.isnan(yz))


@pytest.mark.parametrize("fmt", OF.FORMATS)
@pytest.mark.parametrize("b", [1, 3, 8])
@pytest.mark.parametrize("n,kb", [(67, 4), (9, 56)])
def test_rmsnorm_gemv_unit_gain(fmt, b, n, kb):
    """gamma = NULL (the gain folded into W by the caller): the oracle with a
    gain of ones."""
    k = 256 * kb
    blk = make_blocks(fmt, n, k, seed=27, tid=n + kb)
    x = residual_stream(b, k, 27, b)
    y = run_norm(fmt, OF.pack(fmt, blk), x, None, 1e-5, n, k)
    assert_norm_parity(y, OF.dequant(fmt, blk), x, np.ones(k, np.float32), 1e-5, f"{fmt} unit gain B={b}")


@pytest.mark.parametrize("n,k", [(14336, 4096), (1024, 4096)])
@pytest.mark.parametrize("b", [1, 8])
def test_rmsnorm_gemv_folded_gain_full_size(n, k, b):
    """Full size with the gain folded into the weights before quantization
    (W * diag(gamma), C++ quantizer) and gamma = NULL at run time; sampled
    rows against the oracle's unit-gain normalised GEMV of the same bytes."""
    g = gain(k, 28, 0)
    wf = (full_weights(n, k) * g[None, :]).astype(np.float32)
    packed = qg.qquant("q4_k", wf)
    x = residual_stream(b, k, 28, b)
    y = run_norm("q4_k", packed, x, None, 1e-5, n, k)
    rows = sampled_rows(n, 5 * n + b)
    sub = OF.quantize("q4_k", wf[rows])
    check_sampled_bytes("q4_k", packed, sub, rows, n, k)
    assert_norm_parity(y[:, rows], OF.dequant("q4_k", sub), x, np.ones(k, np.float32), 1e-5, f"folded {n}x{k} B={b}")


def test_rmsnorm_gemv_deterministic():
    n, k = 300, 4096
    blk = make_blocks("q4_k", n, k, seed=25)
    packed = dev(OF.pack("q4_k", blk))
    x, g = dev(residual_stream(2, k, 25, 1)), dev(gain(k, 25, 2))
    ys = []
    for _ in range(3):
        y = torch.empty((2, n), device="cuda")
        qg.qgemv_rmsnorm("q4_k", packed, x, g, 1e-6, y, n, k, 2)
        ys.append(y)
    torch.cuda.synchronize()
    assert all(torch.equal(ys[0], t) for t in ys[1:])


@pytest.mark.parametrize("n,k", [(14336, 4096), (4096, 4096), (1024, 4096)])
@pytest.mark.parametrize("fmt", ["q4_k", "q8_0"])
@pytest.mark.parametrize("b", [1, 8])
def test_rmsnorm_gemv_full_size_sampled_rows(fmt, n, k, b):
    """The projections a decode layer feeds from its norms (gate/up, q/o,
    k/v), at full size with the C++ quantizer's buffer; sampled rows are
    re-quantized by the oracle, checked byte for byte, and checked against
    the oracle's normalised GEMV."""
    w = full_weights(n, k)
    packed = qg.qquant(fmt, w)
    x, g = residual_stream(b, k, 26, b), gain(k, 26, 0)
    y = run_norm(fmt, packed, x, g, 1e-5, n, k)
    rows = sampled_rows(n, 3 * n + b)
    sub = OF.quantize(fmt, w[rows])
    check_sampled_bytes(fmt, packed, sub, rows, n, k)
    assert_norm_parity(y[:, rows], OF.dequant(fmt, sub), x, g, 1e-5, f"{fmt} {n}x{k} B={b}")
    assert np.all(np.isfinite(y))


@pytest.mark.parametrize("fmt,with_gain", [("q4_k", True), ("q8_0", False)])
def test_rmsnorm_gemv_max_k(fmt, with_gain):
    """K = 2^26, the GEMV limit, on one 16-row group: a 16 x 4096 matrix,
    x and gamma repeated 2^14 times along K (the planes of one row group
    repeat with the columns).  The RMS of the repeated row equals the small
    row's, so the exact result is 2^14 times the small normalised GEMV; the
    tolerance's relative part scales the same way."""
    rows, k0, reps, b, eps = 16, 4096, 1 << 14, 2, 1e-5
    k = k0 * reps
    w0 = workloads.student_t_weights(rows, k0, 41, 1)
    small = qg.qquant(fmt, w0)
    cb0 = qg.qg_codes_plane_size(fmt, rows, k0)
    np.testing.assert_array_equal(np.concatenate([np.tile(small[:cb0], 2), np.tile(small[cb0:], 2)]),
                                  qg.qquant(fmt, np.tile(w0, (1, 2))))
    cb, total = qg.qg_codes_plane_size(fmt, rows, k), qg.qg_packed_size(fmt, rows, k)
    assert cb == reps * cb0 and total == reps * small.size
    big = torch.empty(total, dtype=torch.uint8, device="cuda")
    small_d = dev(small)
    big[:cb].view(reps, cb0).copy_(small_d[:cb0].expand(reps, cb0))
    big[cb:].view(reps, -1).copy_(small_d[cb0:].expand(reps, small.size - cb0))
    x0 = residual_stream(b, k0, 41, 2)
    g0 = gain(k0, 41, 3) if with_gain else np.ones(k0, np.float32)
    x = dev(x0).repeat(1, reps)
    g = dev(g0).repeat(reps) if with_gain else None
    y_d = torch.full((b, rows), float("nan"), device="cuda")
    qg.qgemv_rmsnorm(fmt, big, x, g, eps, y_d, rows, k, b)
    torch.cuda.synchronize()
    y = y_d.cpu().numpy().astype(np.float64)
    del big, x, g
    torch.cuda.empty_cache()
    w_deq = OF.dequant_packed(fmt, small, rows, k0)
    err = np.abs(y - reps * ON.gemv_rmsnorm_ref(w_deq, x0, g0, eps))
    tol = reps * ON.tolerance(w_deq, x0, g0, eps)
    assert np.all(err <= tol), f"{fmt}: worst |err|/tol = {np.max(err / tol):.3g}"
