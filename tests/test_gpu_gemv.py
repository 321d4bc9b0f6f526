"""GPU parity of the GEMV and dequant kernels against the oracle, through the
C ABI.  Inputs come from the seeded generators; packed weights and expected
values come from the oracle (or, at full size, from the C++ quantizer whose
sampled rows are first checked byte-for-byte against the oracle's)."""
import functools

import numpy as np
import pytest

import block_quantized_decode_qgemv_amd as qg
import workloads
from oracle import formats as OF
from oracle import gemv as OG

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def make_blocks(fmt, n, k, seed=0, tid=0):
    if fmt == "tern":
        return OF.tern_from_codes(workloads.ternary_codes(n, k, seed, tid),
                                  workloads.scale_bits_f16((n, k // 128), seed, tid + 1))
    if fmt == "bin":
        return OF.bin_from_codes(workloads.binary_codes(n, k, seed, tid),
                                 workloads.scale_bits_f16((n, k // 128), seed, tid + 1))
    if fmt == "bin8":
        return OF.bin8_from_codes(workloads.binary_codes(n, k, seed, tid),
                                  workloads.scale_bits_f16((n, k // 128), seed, tid + 1))
    if fmt == "tern3":
        return OF.tern3_from_codes(workloads.ternary_codes(n, k, seed, tid),
                                   workloads.scale_bits_f16((n, k // 64), seed, tid + 1))
    return OF.quantize(fmt, workloads.student_t_weights(n, k, seed, tid))


def run_gemv(fmt, packed, x, n, k):
    b = x.shape[0]
    w_d = dev(packed)
    x_d = dev(x)
    y_d = torch.full((b, n), float("nan"), device="cuda")
    qg.qgemv(fmt, w_d, x_d, y_d, n, k, b)
    torch.cuda.synchronize()
    return y_d.cpu().numpy()


def assert_parity(y, w_deq, x, label):
    ok, ratio, idx = OG.check(y, w_deq, x)
    assert ok, f"{label}: worst |err|/tol = {ratio:.3g} at {idx}"


SHAPES = [(1, 1), (3, 2), (67, 4), (130, 16), (9, 56)]  # (N, K in blocks of 256)


@pytest.mark.parametrize("fmt", OF.FORMATS)
@pytest.mark.parametrize("n,kb", SHAPES)
def test_dequant_bit_exact(fmt, n, kb):
    k = 256 * kb
    blk = make_blocks(fmt, n, k, seed=1, tid=n)
    packed = OF.pack(fmt, blk)
    out = torch.full((n, k), float("nan"), device="cuda")
    qg.qg_dequant(fmt, dev(packed), out, n, k)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = OF.dequant(fmt, blk)
    np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("fmt", OF.FORMATS)
def test_dequant_subnormal_and_signed_scales(fmt):
    """fp16 subnormal and negative scales must decode exactly (no flushing);
    bin8: fp32 subnormal, negative and zero-step per-row (base, step) pairs."""
    n, k = 4, 512
    blk = make_blocks(fmt, n, k, seed=2)
    if fmt == "bin8":
        blk["base"] = np.array([1e-40, -0.75, 3.0, 0.0], np.float32)
        blk["step"] = np.array([1e-41, 2.0 ** -10, 0.0, -1e-3], np.float32)
        out = torch.empty((n, k), device="cuda")
        qg.qg_dequant(fmt, dev(OF.pack(fmt, blk)), out, n, k)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), OF.dequant(fmt, blk).view(np.uint32))
        return
    blk["d"] = blk["d"].copy()
    blk["d"][0] = 0x0001          # smallest fp16 subnormal
    blk["d"][1] = 0x03FF          # largest fp16 subnormal
    blk["d"][2] = blk["d"][2] | 0x8000  # negative scale
    if "dmin" in blk:
        blk["dmin"] = blk["dmin"].copy()
        blk["dmin"][3] = 0x0200
    if "m" in blk:
        blk["m"] = blk["m"].copy()
        blk["m"][3] = 0x8001
    packed = OF.pack(fmt, blk)
    out = torch.empty((n, k), device="cuda")
    qg.qg_dequant(fmt, dev(packed), out, n, k)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), OF.dequant(fmt, blk).view(np.uint32))


@pytest.mark.parametrize("fmt", OF.FORMATS)
@pytest.mark.parametrize("b", [1, 2, 4, 8])
@pytest.mark.parametrize("n,kb", SHAPES)
def test_gemv_parity(fmt, b, n, kb):
    k = 256 * kb
    blk = make_blocks(fmt, n, k, seed=3, tid=7 * n + kb)
    x = workloads.normal((b, k), 3, 1000 + b)
    y = run_gemv(fmt, OF.pack(fmt, blk), x, n, k)
    assert_parity(y, OF.dequant(fmt, blk), x, f"{fmt} B={b} N={n} K={k}")


@pytest.mark.parametrize("fmt", OF.FORMATS)
@pytest.mark.parametrize("b", [1, 2, 4, 8])
def test_gemv_widest_workgroup(fmt, b):
    """K = 16384 gives the register-x kernel its widest workgroup (16 waves,
    one per SIMD slot at low occupancy, where back-to-back issue of a wave's
    instructions is most likely) at small batches, and 8 waves with several
    K slices at the larger ones; 33 rows leave a one-row last group."""
    n, k = 33, 16384
    blk = make_blocks(fmt, n, k, seed=8, tid=b)
    x = workloads.normal((b, k), 8, 100 + b)
    y = run_gemv(fmt, OF.pack(fmt, blk), x, n, k)
    assert_parity(y, OF.dequant(fmt, blk), x, f"{fmt} B={b} N={n} K={k}")


@pytest.mark.parametrize("fmt", OF.FORMATS)
@pytest.mark.parametrize("b", [3, 5, 6, 7])
def test_gemv_odd_batches(fmt, b):
    """Every batch size has its own kernel instance (with fewer code units per
    lane part as the batch grows)."""
    n, k = 45, 2048
    blk = make_blocks(fmt, n, k, seed=9, tid=b)
    x = workloads.normal((b, k), 9, 300 + b)
    y = run_gemv(fmt, OF.pack(fmt, blk), x, n, k)
    assert_parity(y, OF.dequant(fmt, blk), x, f"{fmt} B={b} N={n} K={k}")


@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "q4_1"])
@pytest.mark.parametrize("k", [32, 96, 160, 4064])
def test_gemv_short_blocks(fmt, k):
    """32-weight formats at K that is not a multiple of 256 (ragged chunk tail)."""
    n = 37
    blk = make_blocks(fmt, n, k, seed=4, tid=k)
    x = workloads.normal((3, k), 4, k)
    y = run_gemv(fmt, OF.pack(fmt, blk), x, n, k)
    assert_parity(y, OF.dequant(fmt, blk), x, f"{fmt} K={k}")


@pytest.mark.parametrize("fmt", ["tern", "bin", "bin8"])
@pytest.mark.parametrize("k", [128, 384, 1152, 2176, 4224])
@pytest.mark.parametrize("b", [1, 3, 8])
def test_gemv_odd_unit_counts(fmt, k, b):
    """128-weight formats at K = 128 * odd: an odd number of blocks per row, so
    parts of two units end half outside the row and meta rows end in a short
    unit (bin8: one byte per block)."""
    n = 37
    blk = make_blocks(fmt, n, k, seed=12, tid=k + b)
    x = workloads.normal((b, k), 12, k + b)
    y = run_gemv(fmt, OF.pack(fmt, blk), x, n, k)
    assert_parity(y, OF.dequant(fmt, blk), x, f"{fmt} B={b} K={k}")


@pytest.mark.parametrize("k", [256, 768, 1280, 2304, 4352])
@pytest.mark.parametrize("b", [1, 2, 3, 5, 8])
def test_tern3_odd_block_counts(k, b):
    """tern3 at K = 256 * odd: rows of whole-block parts (batch 1, 2) and of
    half-block parts (batch 3 and up) that end inside a slice, and meta rows
    (12 bytes per block) ending in a short unit."""
    n = 37
    blk = make_blocks("tern3", n, k, seed=14, tid=k + b)
    x = workloads.normal((b, k), 14, k + b)
    y = run_gemv("tern3", OF.pack("tern3", blk), x, n, k)
    assert_parity(y, OF.dequant("tern3", blk), x, f"tern3 B={b} K={k}")


@pytest.mark.parametrize("fmt", OF.FORMATS)
def test_gemv_integer_exact(fmt):
    """Power-of-two scales and small-integer activations: every product and
    partial sum is exact in fp32, so the result must equal the oracle exactly."""
    g = np.random.default_rng(6)
    n, k = 33, 1024
    blk = make_blocks(fmt, n, k, seed=6)
    if fmt == "bin8":  # scales 0.5 + c/256 for the random codes c: exact in fp32
        blk["base"] = np.full(n, 0.5, np.float32)
        blk["step"] = np.full(n, 1 / 256, np.float32)
    else:
        blk["d"] = np.full_like(blk["d"], 0x3C00)      # 1.0
    if "dmin" in blk:
        blk["dmin"] = np.full_like(blk["dmin"], 0x3800)  # 0.5
    if "m" in blk:
        blk["m"] = np.full_like(blk["m"], 0xC000)  # -2.0
    x = g.integers(-3, 4, size=(2, k)).astype(np.float32)
    y = run_gemv(fmt, OF.pack(fmt, blk), x, n, k)
    want = OG.gemv_ref(OF.dequant(fmt, blk), x)
    np.testing.assert_array_equal(y.astype(np.float64), want)


@pytest.mark.parametrize("fmt", OF.FORMATS)
def test_gemv_deterministic(fmt):
    n, k = 515, 4096
    blk = make_blocks(fmt, n, k, seed=7)
    x = workloads.normal((1, k), 7)
    w_d, x_d = dev(OF.pack(fmt, blk)), dev(x)
    y1 = torch.empty((1, n), device="cuda")
    y2 = torch.empty((1, n), device="cuda")
    qg.qgemv(fmt, w_d, x_d, y1, n, k, 1)
    qg.qgemv(fmt, w_d, x_d, y2, n, k, 1)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


def test_single_q4k_gemv_seed0():
    """The single Q4_K GEMV case: W 1024x1024 then x from one default_rng(0)."""
    w, x = workloads.single_q4k_case(1024, 1024, seed=0)
    blk = OF.quantize("q4_k", w)
    packed = OF.pack("q4_k", blk)
    np.testing.assert_array_equal(qg.qquant("q4_k", w), packed)
    y = run_gemv("q4_k", packed, x, 1024, 1024)
    assert_parity(y, OF.dequant("q4_k", blk), x, "q4_k 1024x1024 seed 0")


@functools.lru_cache(maxsize=4)
def full_weights(n, k):
    return workloads.student_t_weights(n, k, seed=0, tensor_id=n)


@functools.lru_cache(maxsize=4)
def full_low_bit_codes(fmt, n, k):
    gen = workloads.ternary_codes if fmt in ("tern", "tern3") else workloads.binary_codes
    return gen(n, k, 11, n), workloads.scale_bits_f16((n, k // (64 if fmt == "tern3" else 128)), 11, n + 1)


def sampled_rows(n, salt):
    return np.unique(np.concatenate([[0, 1, n - 1], np.random.default_rng(salt).choice(n, 253, replace=False)]))


def check_sampled_rows(fmt, packed, sub, rows, n, k, x, y):
    """Rows `rows` of the full device buffer `packed` must equal, byte for byte,
    the oracle's packing of the blocks `sub` of those rows; their outputs are
    checked against the oracle."""
    check_sampled_bytes(fmt, packed, sub, rows, n, k)
    assert_parity(y[:, rows], OF.dequant(fmt, sub), x, f"{fmt} {n}x{k} B={x.shape[0]}")
    assert np.all(np.isfinite(y))


def check_sampled_bytes(fmt, packed, sub, rows, n, k):
    """Rows `rows` of the full buffer `packed` equal the oracle's packing of `sub`."""
    spec = OF.SPECS[fmt]
    cpr = (k // spec.block) * spec.code_bytes
    mpr = (k // spec.block) * spec.meta_bytes
    cp = OF.codes_plane_size(fmt, n, k)
    codes_rows = OF.deinterleave_rows(packed[:cp], n, cpr)
    meta_rows = OF.deinterleave_rows(packed[cp:cp + n * mpr], n, mpr)
    sub_packed = OF.pack(fmt, sub)
    scp = OF.codes_plane_size(fmt, len(rows), k)
    np.testing.assert_array_equal(codes_rows[rows], OF.deinterleave_rows(sub_packed[:scp], len(rows), cpr))
    np.testing.assert_array_equal(meta_rows[rows],
                                  OF.deinterleave_rows(sub_packed[scp:scp + len(rows) * mpr], len(rows), mpr))


@pytest.mark.parametrize("n,k", [(4096, 4096), (14336, 4096)])
@pytest.mark.parametrize("fmt", ["q8_0", "q4_0", "q4_1", "q4_k"])
@pytest.mark.parametrize("b", [1, 8])
def test_full_size_sampled_rows(fmt, n, k, b):
    """Full-size GEMV (the launch the bench times); the device buffer comes from
    the C++ quantizer, and sampled rows are re-quantized by the oracle, checked
    byte-for-byte, and used for the expected outputs."""
    w = full_weights(n, k)
    packed = qg.qquant(fmt, w)
    x = workloads.normal((b, k), 0, 50 + b)
    y = run_gemv(fmt, packed, x, n, k)
    rows = sampled_rows(n, n + b)
    check_sampled_rows(fmt, packed, OF.quantize(fmt, w[rows]), rows, n, k, x, y)


@pytest.mark.parametrize("n,k", [(12288, 4096), (4096, 12288)])
@pytest.mark.parametrize("fmt", ["q2_k", "tern", "bin", "bin8", "tern3"])
@pytest.mark.parametrize("b", [1, 4, 8])
def test_full_size_low_bit_sampled_rows(fmt, n, k, b):
    """The low-bit formats at the bench's full sizes: Q2_K from the C++
    quantizer, tern and bin from the C++ packers over seeded codes; sampled
    rows as in the full-size test.  At batch 8 on 12288 rows the launcher
    halves the waves per workgroup for occupancy."""
    x = workloads.normal((b, k), 0, 60 + b)
    rows = sampled_rows(n, n + 7 * b)
    if fmt == "q2_k":
        w = full_weights(n, k)
        packed = qg.qquant(fmt, w)
        sub = OF.quantize(fmt, w[rows])
    else:
        codes, scales = full_low_bit_codes(fmt, n, k)
        if fmt == "tern":
            packed = qg.qpack_tern(codes, scales)
            sub = OF.tern_from_codes(codes[rows], scales[rows])
        elif fmt == "bin":
            packed = qg.qpack_bin(codes, scales)
            sub = OF.bin_from_codes(codes[rows], scales[rows])
        elif fmt == "tern3":
            packed = qg.qpack_tern3(codes, scales)
            sub = OF.tern3_from_codes(codes[rows], scales[rows])
        else:
            packed = qg.qpack_bin8(codes, scales)
            sub = OF.bin8_from_codes(codes[rows], scales[rows])
    y = run_gemv(fmt, packed, x, n, k)
    if fmt == "bin8":  # the per-row plane after the meta plane, row by row
        tail = packed[-8 * n:].view("<f4").reshape(n, 2)
        np.testing.assert_array_equal(tail[rows, 0], sub["base"])
        np.testing.assert_array_equal(tail[rows, 1], sub["step"])
    check_sampled_rows(fmt, packed, sub, rows, n, k, x, y)


@pytest.mark.parametrize("n,k", [(1024, 4096), (4096, 14336)])
def test_decode_step_shapes_sampled_rows(n, k):
    """The 8B step's k/v and down shapes (Q4_K, batch 1) at full size, sampled
    rows against the oracle as in the full-size test."""
    test_full_size_sampled_rows("q4_k", n, k, 1)


ALIASES = {"q8_0": "qgemv_q8_0", "q4_0": "qgemv_q4_0", "q4_1": "qgemv_q4_1", "q4_k": "qgemv_q4k",
           "q2_k": "qgemv_q2k", "tern": "qgemv_tern", "bin": "qgemv_bin", "bin8": "qgemv_bin8",
           "tern3": "qgemv_tern3"}


@pytest.mark.parametrize("fmt", OF.FORMATS)
def test_per_format_entry_points_match_qgemv(fmt):
    """Each per-format entry point is qgemv with its format: same bits."""
    n, k, b = 70, 1024, 3
    blk = make_blocks(fmt, n, k, seed=13)
    w_d, x_d = dev(OF.pack(fmt, blk)), dev(workloads.normal((b, k), 13, 1))
    y1 = torch.empty((b, n), device="cuda")
    y2 = torch.empty((b, n), device="cuda")
    qg.qgemv(fmt, w_d, x_d, y1, n, k, b)
    getattr(qg, ALIASES[fmt])(w_d, x_d, y2, n, k, b)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("fmt,n,k,b", [("q4_k", 57344, 4096, 1), ("q8_0", 64, 65536, 2), ("q4_k", 48, 131072, 3),
                                       ("bin8", 40, 65536, 8), ("tern3", 40, 65536, 8), ("tern3", 24, 131072, 1)])
def test_large_shapes(fmt, n, k, b):
    """Far beyond the bench's shapes: 57344 rows (3584 row groups, several
    rounds of workgroups per compute unit) and K up to 131072 (many K slices
    per workgroup); sampled rows (all rows when few) against the oracle."""
    x = workloads.normal((b, k), 37, n + k)
    if fmt == "bin8":
        bits, sc = workloads.binary_codes(n, k, 37, 1), workloads.scale_bits_f16((n, k // 128), 37, 2)
        packed = qg.qpack_bin8(bits, sc)
        rows = np.arange(n)
        sub = OF.bin8_from_codes(bits, sc)
    elif fmt == "tern3":
        codes, sc = workloads.ternary_codes(n, k, 37, 1), workloads.scale_bits_f16((n, k // 64), 37, 2)
        packed = qg.qpack_tern3(codes, sc)
        rows = np.arange(n)
        sub = OF.tern3_from_codes(codes, sc)
    else:
        w = workloads.student_t_weights(n, k, 37, n)
        packed = qg.qquant(fmt, w, n_threads=16)
        rows = sampled_rows(n, n + k) if n > 256 else np.arange(n)
        sub = OF.quantize(fmt, w[rows])
    y = run_gemv(fmt, packed, x, n, k)
    check_sampled_rows(fmt, packed, sub, rows, n, k, x, y)


@pytest.mark.parametrize("fmt,reps,k,b", [("q8_0", 5120, 16384, 2), ("q4_k", 10240, 16384, 1)])
def test_over_4gib_matrix(fmt, reps, k, b):
    """A matrix of 5.7-6 GB, so both planes and the meta plane's start lie
    past 2^32 bytes: a 64-row matrix from the C++ quantizer tiled `reps`
    times on the device.  Each plane stores row groups in order, so tiling
    each plane gives the matrix whose row r is row r mod 64 (checked on the
    host at 4 copies against the quantizer of the tiled weights); every
    output row is checked against the oracle's GEMV of the 64 rows."""
    n0 = 64
    w0 = workloads.student_t_weights(n0, k, 38, k)
    small = qg.qquant(fmt, w0)
    cb0 = qg.qg_codes_plane_size(fmt, n0, k)
    np.testing.assert_array_equal(
        np.concatenate([np.tile(small[:cb0], 4), np.tile(small[cb0:], 4)]),
        qg.qquant(fmt, np.tile(w0, (4, 1))))
    n = n0 * reps
    cb, total = qg.qg_codes_plane_size(fmt, n, k), qg.qg_packed_size(fmt, n, k)
    assert cb == reps * cb0 and total == reps * small.size and total > (1 << 32) + cb0
    big = torch.empty(total, dtype=torch.uint8, device="cuda")
    small_d = dev(small)
    big[:cb].view(reps, cb0).copy_(small_d[:cb0].expand(reps, cb0))
    big[cb:].view(reps, -1).copy_(small_d[cb0:].expand(reps, small.size - cb0))
    x = workloads.normal((b, k), 38, 1)
    y_d = torch.full((b, n), float("nan"), device="cuda")
    qg.qgemv(fmt, big, dev(x), y_d, n, k, b)
    torch.cuda.synchronize()
    y = y_d.cpu().numpy().reshape(b, reps, n0).astype(np.float64)
    del big
    torch.cuda.empty_cache()
    w_deq = OF.dequant_packed(fmt, small, n0, k)
    err = np.abs(y - OG.gemv_ref(w_deq, x)[:, None, :])
    tol = OG.tolerance(w_deq, x)[:, None, :]
    worst = np.unravel_index(int(np.argmax(err / tol)), err.shape)
    assert np.all(err <= tol), f"{fmt}: |err|/tol = {err[worst] / tol[worst]:.3g} at (b, copy, row) {worst}"


@pytest.mark.parametrize("fmt", ["q8_0", "q4_k"])
def test_max_k_one_row_group(fmt):
    """K = 2^26, the GEMV limit, on one 16-row group (in-group offsets up to
    2^30 bytes, 32-bit by design): a 16 x 4096 matrix repeated 2^14 times
    along K.  For one row group each plane is the row's units in order, so
    repeating the planes repeats the columns (checked on the host at 3
    copies); with x repeated the same way the exact result is 2^14 times the
    small one, and the accuracy bound scales the same way."""
    rows, k0, reps, b = 16, 4096, 1 << 14, 2
    k = k0 * reps
    w0 = workloads.student_t_weights(rows, k0, 40, 1)
    small = qg.qquant(fmt, w0)
    cb0 = qg.qg_codes_plane_size(fmt, rows, k0)
    np.testing.assert_array_equal(np.concatenate([np.tile(small[:cb0], 3), np.tile(small[cb0:], 3)]),
                                  qg.qquant(fmt, np.tile(w0, (1, 3))))
    cb, total = qg.qg_codes_plane_size(fmt, rows, k), qg.qg_packed_size(fmt, rows, k)
    assert cb == reps * cb0 and total == reps * small.size
    big = torch.empty(total, dtype=torch.uint8, device="cuda")
    small_d = dev(small)
    big[:cb].view(reps, cb0).copy_(small_d[:cb0].expand(reps, cb0))
    big[cb:].view(reps, -1).copy_(small_d[cb0:].expand(reps, small.size - cb0))
    x0 = workloads.normal((b, k0), 40, 2)
    x = dev(x0).repeat(1, reps)
    y_d = torch.full((b, rows), float("nan"), device="cuda")
    qg.qgemv(fmt, big, x, y_d, rows, k, b)
    torch.cuda.synchronize()
    y = y_d.cpu().numpy().astype(np.float64)
    del big, x
    torch.cuda.empty_cache()
    w_deq = OF.dequant_packed(fmt, small, rows, k0)
    err = np.abs(y - reps * OG.gemv_ref(w_deq, x0))
    tol = reps * OG.tolerance(w_deq, x0)
    assert np.all(err <= tol), f"{fmt}: worst |err|/tol = {np.max(err / tol):.3g}"
