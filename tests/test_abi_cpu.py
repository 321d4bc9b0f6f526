"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/qgemv.h declares, validates arguments before any
launch, and reports sizes that match the oracle's layout."""
import os
import re
import subprocess

import numpy as np
import pytest

import block_quantized_decode_qgemv_amd as qg
from oracle import formats as OF

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemv.h")


def _declared():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, flags=re.M))


def test_library_exports_every_declared_symbol():
    lib = qg.load()
    declared = _declared()
    assert declared == set(qg.EXPORTED_SYMBOLS)
    for name in declared:
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", qg.lib_path()], capture_output=True, text=True, check=True)
    exported = {line.split()[-1] for line in out.stdout.splitlines() if " T " in line}
    assert declared <= exported


def test_version_and_strerror():
    assert "gfx950" in qg.qg_version()
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert qg.qg_strerror(code)


@pytest.mark.parametrize("fmt", OF.FORMATS)
def test_sizes_match_oracle(fmt):
    for n, k in ((1, 256), (3, 1024), (4096, 4096), (14336, 4096), (4096, 14336)):
        assert qg.qg_packed_size(fmt, n, k) == OF.packed_size(fmt, n, k)
        assert qg.qg_codes_plane_size(fmt, n, k) == OF.codes_plane_size(fmt, n, k)
        assert qg.qg_codes_plane_offset(fmt, n, k) == OF.codes_plane_size(fmt, n, k)
    assert qg.qg_block_size(fmt) == OF.SPECS[fmt].block
    assert qg.qg_packed_size(fmt, 0, 256) == 0
    assert qg.qg_packed_size(fmt, 4, OF.SPECS[fmt].block + 1) == 0
    assert qg.qg_packed_size(99, 4, 256) == 0


# The cases below hand the library fake (aligned, non-null) device pointers
# with arguments that must be rejected before any launch.  They are host-logic
# tests for a machine without a GPU and are skipped where a GPU is present.

def _gpu_present():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


nogpu = pytest.mark.skipif(_gpu_present(), reason="validation-only tests use fake device pointers")

P = 0x10000  # fake 16-byte aligned pointer value


@nogpu
@pytest.mark.parametrize("args,code", [
    (dict(fmt=3, n=0, k=256, b=1), -2),          # N < 1
    (dict(fmt=3, n=4, k=128, b=1), -2),          # K not a multiple of 256
    (dict(fmt=0, n=4, k=48, b=1), -2),           # K not a multiple of 32
    (dict(fmt=3, n=4, k=256, b=0), -4),          # B < 1
    (dict(fmt=3, n=4, k=256, b=9), -4),          # B > 8
    (dict(fmt=9, n=4, k=256, b=1), -1),          # unknown format
    (dict(fmt=3, n=1 << 31, k=256, b=1), -2),    # N beyond int
    (dict(fmt=-1, n=4, k=256, b=1), -1),
    (dict(fmt=3, n=4, k=256, b=1, w=0), -1),     # null w
    (dict(fmt=3, n=4, k=256, b=1, x=0), -1),     # null x
    (dict(fmt=3, n=4, k=256, b=1, y=0), -1),     # null y
    (dict(fmt=3, n=4, k=1 << 27, b=1), -2),      # K beyond the GEMV limit
    (dict(fmt=3, n=4, k=256, b=1, w=P + 8), -3),  # misaligned w
    (dict(fmt=3, n=4, k=256, b=1, x=P + 4), -3),  # misaligned x
    (dict(fmt=3, n=4, k=256, b=1, y=P + 2), -3),  # misaligned y
    (dict(fmt=3, n=4, k=256, b=2, x=P + 1024, y=P + 1024 + 2040), -1),  # y overlaps the end of x
    (dict(fmt=3, n=4, k=256, b=1, w=P + 4096, y=P + 4096 + 560), -1),   # y overlaps the end of w (576 B)
])
def test_gemv_validation(args, code):
    lib = qg.load()
    rc = lib.qgemv(args["fmt"], args.get("w", P), args.get("x", P), args.get("y", P),
                   args["n"], args["k"], args["b"], None, 0, None)
    assert rc == code, qg.qg_last_error()
    assert qg.qg_last_error()


@nogpu
def test_gemv_rmsnorm_validation():
    import ctypes

    lib = qg.load()

    big = 1 << 24  # distinct, non-overlapping fake buffers

    def call(fmt=3, w=P, x=P + big, gamma=P + 2 * big, eps=1e-6, y=P + 3 * big, n=4, k=256, b=1):
        return lib.qgemv_rmsnorm(fmt, w, x, gamma, ctypes.c_float(eps), y, n, k, b, None)

    assert call(gamma=P + 4) == -3
    assert call(gamma=None, eps=-1e-6) == -4   # unit gain: the other checks still apply
    assert call(eps=-1e-6) == -4
    assert call(eps=float("nan")) == -4
    assert call(eps=float("inf")) == -4
    assert call(k=128) == -2            # the plain GEMV's checks come first
    assert call(b=9) == -4
    assert call(x=None) == -1
    assert call(y=P + 2 * big + 1008) == -1   # y overlaps the end of gamma (1 KiB)
    assert qg.qg_last_error()


@nogpu
def test_moe_rmsnorm_validation():
    import ctypes

    lib = qg.load()
    ws = qg.moe_expert_ffn_workspace_size(2, 16, 512, 256, 4)

    big = 1 << 24  # distinct, non-overlapping fake buffers
    wsp = P + 7 * big

    def call(fmt=3, gamma=P + 6 * big, eps=1e-6, x=P + big, t=2, ws_bytes=ws):
        return lib.moe_expert_ffn_rmsnorm(fmt, P, P, 16, 512, 256, 4, x, gamma, ctypes.c_float(eps), P + 2 * big,
                                          P + 3 * big, P + 4 * big, t, 0, P + 5 * big, wsp, ws_bytes, None)

    assert call(gamma=P + 4) == -3
    assert call(gamma=None, eps=-1.0) == -4   # unit gain: the other checks still apply
    assert call(eps=-1.0) == -4
    assert call(eps=float("nan")) == -4
    assert call(fmt=0) == -1            # the plain layer's checks come first
    assert call(t=9) == -4
    assert call(ws_bytes=ws - 16) == -4
    assert call(gamma=wsp + 512) == -1   # gamma inside the workspace
    assert call(x=P + 5 * big - 64) == -1  # x overlaps out
    assert qg.qg_last_error()


@nogpu
def test_device_quantizer_validation():
    lib = qg.load()
    assert lib.qquant_device(5, P, 4, 256, P, P, None) == -6          # tern: no quantizer
    assert lib.qquant_device(6, P, 4, 256, P, P, None) == -6          # bin
    assert lib.qquant_device(3, P, 4, 128, P, P, None) == -2          # K off the block grid
    assert lib.qquant_device(3, None, 4, 256, P, P, None) == -1
    assert lib.qquant_device(3, P, 4, 256, P, None, None) == -1       # null status
    assert lib.qquant_device(3, P, 4, 256, P + 8, P, None) == -3      # misaligned out
    ws = qg.qrequant_workspace_size(4, 256)
    assert ws == 4 * 256 * 4
    assert qg.qrequant_workspace_size((1 << 31) - 1, 256) > 0 and qg.qrequant_workspace_size(1 << 31, 256) == 0
    big = 1 << 24
    assert lib.qrequant(3, P, 4, P + big, 4, 256, P + 2 * big, ws - 4, P + 3 * big, None) == -4
    assert lib.qrequant(3, P, 4, P + 16, 4, 256, P + 2 * big, ws, P + 3 * big, None) == -1   # src/dst overlap
    assert lib.qrequant(3, P, 4, P + big, 4, 256, P + big + 16, ws, P + 3 * big, None) == -1  # ws/dst overlap
    assert lib.qrequant(3, P, 5, P + big, 4, 256, P + 2 * big, ws, P + 3 * big, None) == -6  # dst tern
    assert lib.qrequant(9, P, 4, P + big, 4, 256, P + 2 * big, ws, P + 3 * big, None) == -1  # unknown src
    assert lib.qrequant(3, P, 4, P + big, 4, 256, P + 2 * big, ws, P + big + 4, None) == -1  # status in dst
    assert lib.qquant_device(3, P, 4, 256, P + 1024, P + 8192, None) == -1          # out overlaps w (4 KiB)
    assert lib.qquant_device(3, P, 4, 256, P + 8192, P + 8192 + 16, None) == -1     # status in out
    assert qg.qg_last_error()


@nogpu
def test_dequant_validation():
    lib = qg.load()
    assert lib.qg_dequant(3, P, P, 0, 256, None) == -2
    assert lib.qg_dequant(3, None, P, 4, 256, None) == -1
    assert lib.qg_dequant(3, P + 4, P, 4, 256, None) == -3


@nogpu
def test_read_probe_validation():
    lib = qg.load()
    assert lib.qg_hbm_read_probe(None, 16, P, None) == -1
    assert lib.qg_hbm_read_probe(P, 0, P, None) == -2
    assert lib.qg_hbm_read_probe(P, 24, P, None) == -2
    assert lib.qg_hbm_read_probe(P + 4, 32, P, None) == -3


def test_binding_rejects_host_tensors():
    import torch

    w = torch.zeros(qg.qg_packed_size("q4_k", 4, 256), dtype=torch.uint8)
    x = torch.zeros(1, 256)
    y = torch.zeros(1, 4)
    with pytest.raises(TypeError):
        qg.qgemv_q4k(w, x, y, 4, 256)


def test_library_missing_is_loud(tmp_path, monkeypatch):
    monkeypatch.setattr(qg, "_lib", None)
    monkeypatch.setattr(qg, "_HERE", str(tmp_path))
    monkeypatch.setattr(qg, "lib_path", lambda: os.path.join(str(tmp_path), "libqgemv.so"))
    with pytest.raises(qg.QGLibraryMissing):
        qg.load()


# The binding compares every tensor's byte size with what the call reads or
# writes through it, before anything reaches the library.  A stand-in for a
# device tensor (it only answers the questions the binding asks) lets the
# checks run without a GPU.

class _FakeDev:
    is_cuda = True

    def __init__(self, nbytes, dtype):
        import torch

        self.dtype = dtype
        self._esize = torch.empty(0, dtype=dtype).element_size()
        self._numel = nbytes // self._esize

    def is_contiguous(self):
        return True

    def numel(self):
        return self._numel

    def element_size(self):
        return self._esize

    def data_ptr(self):
        # a fake aligned address: every call below fails its size check
        # before the library is entered, so it is never dereferenced
        return P


def _f32(nbytes):
    import torch

    return _FakeDev(nbytes, torch.float32)


def _u8(nbytes):
    import torch

    return _FakeDev(nbytes, torch.uint8)


@pytest.mark.parametrize("short", ["w", "x", "y", "ws"])
def test_binding_rejects_undersized_gemv_tensors(short):
    n, k, b = 40, 512, 3
    size = {"w": qg.qg_packed_size("q4_k", n, k), "x": 4 * b * k, "y": 4 * b * n, "ws": 256}
    args = {name: (_u8 if name in ("w", "ws") else _f32)(nb - (4 if name == short else 0)) for name, nb in size.items()}
    with pytest.raises(ValueError, match=short):
        qg.qgemv("q4_k", args["w"], args["x"], args["y"], n, k, b, ws=args["ws"], ws_bytes=256)
    if short != "ws":
        with pytest.raises(ValueError, match=short):
            qg.qgemv_q4k(args["w"], args["x"], args["y"], n, k, b)


@pytest.mark.parametrize("short", ["w", "x", "gamma", "y"])
def test_binding_rejects_undersized_rmsnorm_tensors(short):
    n, k, b = 16, 256, 2
    size = {"w": qg.qg_packed_size("q8_0", n, k), "x": 4 * b * k, "gamma": 4 * k, "y": 4 * b * n}
    a = {name: (_u8 if name == "w" else _f32)(nb - (4 if name == short else 0)) for name, nb in size.items()}
    with pytest.raises(ValueError, match=short):
        qg.qgemv_rmsnorm("q8_0", a["w"], a["x"], a["gamma"], 1e-6, a["y"], n, k, b)


def test_binding_rejects_undersized_dequant_quant_probe():
    n, k = 32, 256
    with pytest.raises(ValueError, match="out"):
        qg.qg_dequant("q4_0", _u8(qg.qg_packed_size("q4_0", n, k)), _f32(4 * n * k - 4), n, k)
    with pytest.raises(ValueError, match="w"):
        qg.qg_dequant("q4_0", _u8(qg.qg_packed_size("q4_0", n, k) - 1), _f32(4 * n * k), n, k)
    with pytest.raises(ValueError, match="out"):
        qg.qquant_device("q4_k", _f32(4 * n * k), _u8(qg.qg_packed_size("q4_k", n, k) - 16), n, k, _u8(4))
    with pytest.raises(ValueError, match="status"):
        qg.qquant_device("q4_k", _f32(4 * n * k), _u8(qg.qg_packed_size("q4_k", n, k)), n, k, _u8(2))
    ws = qg.qrequant_workspace_size(n, k)
    with pytest.raises(ValueError, match="dst"):
        qg.qrequant("q4_k", _u8(qg.qg_packed_size("q4_k", n, k)), "q2_k", _u8(qg.qg_packed_size("q2_k", n, k) - 1),
                    n, k, _u8(ws), ws, _u8(4))
    with pytest.raises(ValueError, match="workspace"):
        qg.qrequant("q4_k", _u8(qg.qg_packed_size("q4_k", n, k)), "q2_k", _u8(qg.qg_packed_size("q2_k", n, k)),
                    n, k, _u8(ws - 4), ws, _u8(4))
    with pytest.raises(ValueError, match="buf"):
        qg.qg_hbm_read_probe(_u8(1024), 2048, _u8(4))


@pytest.mark.parametrize("short", ["w_gate_up", "w_down", "x", "residual", "router_logits", "shared_gate_logit",
                                   "out", "workspace", "gamma"])
def test_binding_rejects_undersized_moe_tensors(short):
    t, e, h, i, top_k = 2, 6, 256, 256, 2
    ws = qg.moe_expert_ffn_workspace_size(t, e, h, i, top_k)
    size = {"w_gate_up": (e + 1) * qg.qg_packed_size("q4_k", 2 * i, h),
            "w_down": (e + 1) * qg.qg_packed_size("q4_k", h, i),
            "x": 4 * t * h, "residual": 4 * t * h, "router_logits": 4 * t * e, "shared_gate_logit": 4 * t,
            "out": 4 * t * h, "workspace": ws, "gamma": 4 * h}
    a = {name: (_u8 if name in ("w_gate_up", "w_down", "workspace") else _f32)(nb - (4 if name == short else 0))
         for name, nb in size.items()}
    with pytest.raises(ValueError, match=short):
        qg.moe_expert_ffn_rmsnorm("q4_k", a["w_gate_up"], a["w_down"], e, h, i, top_k, a["x"], a["gamma"], 1e-6,
                                  a["residual"], a["router_logits"], a["shared_gate_logit"], t, a["out"],
                                  a["workspace"], ws)
    if short != "gamma":
        with pytest.raises(ValueError, match=short):
            qg.moe_expert_ffn("q4_k", a["w_gate_up"], a["w_down"], e, h, i, top_k, a["x"], a["residual"],
                              a["router_logits"], a["shared_gate_logit"], t, a["out"], a["workspace"], ws)


@pytest.mark.parametrize("packer,codes", [("qpack_tern", np.zeros((3, 256), np.int8)),
                                          ("qpack_bin", np.zeros((3, 256), np.uint8)),
                                          ("qpack_bin8", np.zeros((3, 256), np.uint8))])
def test_packers_check_scale_shape(packer, codes):
    fn = getattr(qg, packer)
    good = np.full((3, 2), 0x3C00, np.uint16)
    assert fn(codes, good).size == qg.qg_packed_size(packer[len("qpack_"):], 3, 256)
    for bad in (np.full((3, 1), 0x3C00, np.uint16), np.full((2, 2), 0x3C00, np.uint16),
                np.full((6,), 0x3C00, np.uint16)):
        with pytest.raises(ValueError, match="scale_bits"):
            fn(codes, bad)
    with pytest.raises(ValueError, match="2-D"):
        fn(codes.reshape(-1), good)
    with pytest.raises(ValueError, match="multiple of 128"):
        fn(np.zeros((3, 200), codes.dtype), good)


def test_moe_workspace_layout_offsets():
    for t, e, h, i, k in ((1, 512, 4096, 1024, 4), (8, 512, 4096, 1024, 4), (3, 16, 512, 256, 2)):
        size = qg.moe_expert_ffn_workspace_size(t, e, h, i, k)
        hs, ho = qg.moe_expert_ffn_workspace_layout(t, e, h, i, k)
        rows = t * k + (t + 1) // 2  # routed (token, slot) pairs plus the shared expert's items, two rows each
        assert hs % 16 == 0 and ho % 16 == 0
        assert hs + 4 * t * (k + 1) <= ho
        assert ho + 4 * 2 * rows * i <= size
    with pytest.raises(qg.QGError):
        qg.moe_expert_ffn_workspace_layout(9, 16, 512, 256, 2)


@nogpu
def test_moe_noalloc_validation():
    lib = qg.load()
    big = 1 << 24

    def call(fmt=3, e=16, h=512, i=256, k=4, t=2, x=P + big, out=P + 5 * big):
        return lib.moe_expert_ffn_noalloc(fmt, P, P, e, h, i, k, x, P + 2 * big, P + 3 * big, P + 4 * big, t, 0,
                                          out, None)

    assert call(fmt=0) == -1
    assert call(t=9) == -4
    assert call(h=300) == -2
    assert call(x=P + 5 * big - 64) == -1      # x overlaps out
    assert call(i=4096, k=8, t=8) == -4        # the layer's workspace exceeds the scratch
    assert qg.qg_last_error()


def test_gemv_workspace_size():
    # split K only from batch 5 and for row-starved shapes (groups * S <= compute units)
    assert qg.qgemv_workspace_size("q4_k", 1024, 4096, 1) == 0
    assert qg.qgemv_workspace_size("q4_k", 1024, 4096, 3) == 0
    assert qg.qgemv_workspace_size("q4_k", 4096, 4096, 8) == 0
    assert qg.qgemv_workspace_size("q4_k", 14336, 4096, 8) == 0
    for fmt in OF.FORMATS:
        size = qg.qgemv_workspace_size(fmt, 1024, 4096, 8)
        assert size in (4 * 8 * 1024 * 4, 2 * 8 * 1024 * 4), size  # 4 splits on a 256-unit chip
    assert qg.qgemv_workspace_size("q4_k", 1024, 4096 + 256, 8) == 0   # K does not split into 256-column pieces
    assert qg.qgemv_workspace_size("q4_k", 1024, 128, 8) == 0          # invalid K
    assert qg.qgemv_workspace_size("q4_k", 1024, 4096, 9) == 0         # invalid B


@nogpu
def test_gemv_splitk_workspace_validation():
    lib = qg.load()
    big = 1 << 24
    n, k, b = 1024, 4096, 8
    ws = qg.qgemv_workspace_size("q4_k", n, k, b)
    assert ws > 0
    # w, x, y and ws apart; ws misaligned / overlapping x: rejected before any launch
    assert lib.qgemv(3, P, P + big, P + 2 * big, n, k, b, P + 3 * big + 4, ws, None) == -3
    assert lib.qgemv(3, P, P + big, P + 2 * big, n, k, b, P + big + 64, ws, None) == -1
    assert qg.qg_last_error()
