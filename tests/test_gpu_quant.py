"""GPU parity of the device quantizer (qquant_device) and re-quantizer
(qrequant) against the oracle's quantizer and packer, byte for byte, through
the C ABI: every quantized format, ragged row groups, meta planes with a
short last unit, the quantizer's special blocks, device-side error reports,
and 4-bit -> 2-bit re-quantization of a full expert matrix."""
import numpy as np
import pytest

import block_quantized_decode_qgemv_amd as qg
import workloads
from oracle import formats as OF

from .test_gpu_gemv import dev, make_blocks

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

QFORMATS = ["q8_0", "q4_0", "q4_1", "q4_k", "q2_k"]


def run_quant(fmt, w):
    n, k = w.shape
    out = torch.full((qg.qg_packed_size(fmt, n, k),), 0xA5, dtype=torch.uint8, device="cuda")
    status = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    qg.qquant_device(fmt, dev(w), out, n, k, status)
    torch.cuda.synchronize()
    return out.cpu().numpy(), int(status.item())


def shapes(fmt):
    blk = OF.SPECS[fmt].block
    if blk == 32:  # K off the 256 grid: meta rows end in a short unit
        return [(1, 32), (37, 96), (130, 4064), (17, 1024)]
    return [(1, 256), (37, 512), (130, 2048), (17, 4096)]


@pytest.mark.parametrize("fmt", QFORMATS)
def test_quant_device_bit_exact(fmt):
    for n, k in shapes(fmt):
        w = workloads.student_t_weights(n, k, 31, n + k)
        got, status = run_quant(fmt, w)
        assert status == 0, qg.qg_strerror(status)
        want = OF.pack(fmt, OF.quantize(fmt, w))
        np.testing.assert_array_equal(got, want, err_msg=f"{fmt} {n}x{k}")


@pytest.mark.parametrize("fmt", QFORMATS)
def test_quant_device_special_blocks(fmt):
    """Zero blocks, constant blocks of either sign, signed zeros, a negative
    extreme, tiny values whose scales are fp16 subnormals, and one huge value
    per block near the fp16 limit."""
    n, k = 20, 512
    w = workloads.student_t_weights(n, k, 32, 0).copy()
    w[0] = 0.0
    w[1] = 0.75
    w[2] = -0.75
    w[3, ::2] = -0.0
    w[4, 5] = -3.0
    w[5] *= np.float32(1e-6)
    w[6] *= np.float32(1e-9)
    w[7, ::32] = 60000.0 * (127.0 / 128.0) if fmt == "q8_0" else 1000.0
    got, status = run_quant(fmt, w)
    assert status == 0, qg.qg_strerror(status)
    np.testing.assert_array_equal(got, OF.pack(fmt, OF.quantize(fmt, w)))


@pytest.mark.parametrize("fmt", QFORMATS)
def test_quant_device_reports_errors(fmt):
    """A non-finite weight reports QG_EINVAL; a scale that overflows fp16
    reports QG_ERANGE; with both the smaller code (QG_ERANGE) stays.  The
    other rows are still quantized exactly."""
    n, k = 33, 512
    w = workloads.student_t_weights(n, k, 33, 0).copy()
    bad = w.copy()
    bad[3, 17] = np.nan
    got, status = run_quant(fmt, bad)
    assert status == -1
    ok_rows = [r for r in range(n) if r != 3]
    want = OF.pack(fmt, OF.quantize(fmt, w))
    # compare the packed bytes of every row but row 3 through the oracle's unpacking
    got_blk = OF.unpack(fmt, got, n, k)
    want_blk = OF.unpack(fmt, want, n, k)
    for key in want_blk:
        np.testing.assert_array_equal(np.asarray(got_blk[key])[ok_rows], np.asarray(want_blk[key])[ok_rows])
    bad[9, 100] = 3.0e9
    _, status = run_quant(fmt, bad)
    assert status == -4


@pytest.mark.parametrize("src,dst", [("q4_k", "q2_k"), ("q8_0", "q4_0"), ("q4_1", "q4_k"), ("tern", "q8_0"),
                                     ("bin", "q4_1"), ("q2_k", "q4_k"), ("tern3", "q2_k")])
def test_requant_bit_exact(src, dst):
    n, k = 45, 1024
    blk = make_blocks(src, n, k, seed=34, tid=n)
    packed = dev(OF.pack(src, blk))
    out = torch.full((qg.qg_packed_size(dst, n, k),), 0x5A, dtype=torch.uint8, device="cuda")
    ws_bytes = qg.qrequant_workspace_size(n, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    status = torch.full((1,), 777, dtype=torch.int32, device="cuda")
    qg.qrequant(src, packed, dst, out, n, k, ws, ws_bytes, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    want = OF.pack(dst, OF.quantize(dst, OF.dequant(src, blk)))
    np.testing.assert_array_equal(out.cpu().numpy(), want)


def test_requant_full_expert_q4k_to_q2k():
    """A full expert gate/up matrix (2048 x 4096 rows of gate and up
    interleaved), quantized to Q4_K by the C++ quantizer, re-quantized to
    Q2_K on the device; every byte against the oracle's Q2_K of the oracle's
    Q4_K decode."""
    n, k = 2048, 4096
    w = workloads.student_t_weights(n, k, 35, 0)
    q4 = qg.qquant("q4_k", w)
    out = torch.empty((qg.qg_packed_size("q2_k", n, k),), dtype=torch.uint8, device="cuda")
    ws_bytes = qg.qrequant_workspace_size(n, k)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    status = torch.zeros((1,), dtype=torch.int32, device="cuda")
    qg.qrequant("q4_k", dev(q4), "q2_k", out, n, k, ws, ws_bytes, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    deq = OF.dequant_packed("q4_k", q4, n, k)
    np.testing.assert_array_equal(out.cpu().numpy(), OF.pack("q2_k", OF.quantize("q2_k", deq)))


@pytest.mark.parametrize("fmt,n,k", [("q4_k", 14336, 4096), ("q8_0", 4096, 4096), ("q2_k", 4096, 14336)])
def test_quant_device_full_size_matches_host_quantizer(fmt, n, k):
    """The device quantizer on a full projection matrix equals the C++ host
    quantizer byte for byte (the host quantizer is pinned to the oracle)."""
    w = workloads.student_t_weights(n, k, 36, n)
    got, status = run_quant(fmt, w)
    assert status == 0
    np.testing.assert_array_equal(got, qg.qquant(fmt, w, n_threads=16))


@pytest.mark.parametrize("fmt,reps,k", [("q8_0", 5120, 16384), ("q4_k", 10240, 16384)])
def test_quant_device_over_4gib_output(fmt, reps, k):
    """A 21-43 GB fp32 matrix (a 64-row matrix tiled on the device) quantized
    on the device into a 5.7-6 GB buffer whose planes run past 2^32 bytes.  Each
    plane stores row groups in order, so the expected buffer is each plane of
    the oracle's packing of the 64 rows repeated `reps` times; every byte is
    compared on the device."""
    n0 = 64
    w0 = workloads.student_t_weights(n0, k, 39, k)
    small = OF.pack(fmt, OF.quantize(fmt, w0))
    cb0 = OF.codes_plane_size(fmt, n0, k)
    n = n0 * reps
    cb, total = qg.qg_codes_plane_size(fmt, n, k), qg.qg_packed_size(fmt, n, k)
    assert cb == reps * cb0 and total == reps * small.size and total > (1 << 32)
    w = dev(w0).repeat(reps, 1)
    out = torch.full((total,), 0xA5, dtype=torch.uint8, device="cuda")
    status = torch.full((1,), 12345, dtype=torch.int32, device="cuda")
    qg.qquant_device(fmt, w, out, n, k, status)
    torch.cuda.synchronize()
    del w
    assert int(status.item()) == 0
    small_d = dev(small)
    assert torch.equal(out[:cb].view(reps, cb0), small_d[:cb0].expand(reps, cb0))
    assert torch.equal(out[cb:].view(reps, -1), small_d[cb0:].expand(reps, small.size - cb0))
