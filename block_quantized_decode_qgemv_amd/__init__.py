"""Python binding for libqgemv.so, the block-quantized decode GEMV library.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/qgemv.h``.  Device arguments
are torch CUDA (HIP) tensors or raw integer device pointers; host arguments
of the reference quantizer are numpy arrays.  ``stream=None`` means torch's
current stream on the current device.

Importing this package does not load the library; the first call does, and
raises ``QGLibraryMissing`` if it was not built
(``python -m block_quantized_decode_qgemv_amd.build``).  There is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

__all__ = [
    "FORMATS", "QG_MOE_RENORM", "QG_MOE_NOALLOC_SCRATCH_BYTES", "QGError", "QGLibraryMissing", "lib_path", "load",
    "qg_packed_size", "qg_codes_plane_size", "qg_codes_plane_offset", "qg_block_size", "qgemv_workspace_size",
    "qgemv", "qgemv_q8_0", "qgemv_q4_0", "qgemv_q4_1", "qgemv_q4k", "qgemv_q2k",
    "qgemv_tern", "qgemv_bin", "qgemv_bin8", "qgemv_tern3", "qgemv_rmsnorm", "qg_dequant", "qquant", "qquant_device", "qrequant_workspace_size", "qrequant",
    "qpack_tern", "qpack_bin", "qpack_bin8", "qpack_tern3",
    "moe_expert_ffn_workspace_size", "moe_expert_ffn_workspace_layout", "moe_expert_ffn", "moe_expert_ffn_noalloc", "moe_expert_ffn_rmsnorm", "qg_strerror", "qg_last_error",
    "qg_version", "EXPORTED_SYMBOLS",
]

QG_MOE_NOALLOC_SCRATCH_BYTES = 2 << 20  # the no-allocation MoE entry point's device scratch (qgemv.h)
FORMATS = {"q8_0": 0, "q4_0": 1, "q4_1": 2, "q4_k": 3, "q2_k": 4, "tern": 5, "bin": 6, "bin8": 7, "tern3": 8}
QG_MOE_RENORM = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libqgemv.so"
_lock = threading.Lock()
_lib = None

_i32, _i64, _u32, _sz, _vp, _cp = (ctypes.c_int, ctypes.c_int64, ctypes.c_uint, ctypes.c_size_t,
                                   ctypes.c_void_p, ctypes.c_char_p)
_GEMV_ARGS = [_vp, _vp, _vp, _i64, _i64, _i32, _vp, _sz, _vp]

# name -> (restype, argtypes); the same set include/qgemv.h declares
_SIGNATURES = {
    "qg_packed_size": (_sz, [_i32, _i64, _i64]),
    "qg_codes_plane_size": (_sz, [_i32, _i64, _i64]),
    "qg_codes_plane_offset": (_sz, [_i32, _i64, _i64]),
    "qg_block_size": (_i32, [_i32]),
    "qgemv_workspace_size": (_sz, [_i32, _i64, _i64, _i32]),
    "qgemv": (_i32, [_i32] + _GEMV_ARGS),
    "qgemv_q8_0": (_i32, _GEMV_ARGS),
    "qgemv_q4_0": (_i32, _GEMV_ARGS),
    "qgemv_q4_1": (_i32, _GEMV_ARGS),
    "qgemv_q4k": (_i32, _GEMV_ARGS),
    "qgemv_q2k": (_i32, _GEMV_ARGS),
    "qgemv_tern": (_i32, _GEMV_ARGS),
    "qgemv_bin": (_i32, _GEMV_ARGS),
    "qgemv_bin8": (_i32, _GEMV_ARGS),
    "qgemv_tern3": (_i32, _GEMV_ARGS),
    "qgemv_rmsnorm": (_i32, [_i32, _vp, _vp, _vp, ctypes.c_float, _vp, _i64, _i64, _i32, _vp]),
    "qg_dequant": (_i32, [_i32, _vp, _vp, _i64, _i64, _vp]),
    "qquant": (_i32, [_i32, _vp, _i64, _i64, _vp, _i32]),
    "qquant_device": (_i32, [_i32, _vp, _i64, _i64, _vp, _vp, _vp]),
    "qrequant_workspace_size": (_sz, [_i64, _i64]),
    "qrequant": (_i32, [_i32, _vp, _i32, _vp, _i64, _i64, _vp, _sz, _vp, _vp]),
    "qpack_tern": (_i32, [_vp, _vp, _i64, _i64, _vp]),
    "qpack_bin": (_i32, [_vp, _vp, _i64, _i64, _vp]),
    "qpack_bin8": (_i32, [_vp, _vp, _i64, _i64, _vp]),
    "qpack_tern3": (_i32, [_vp, _vp, _i64, _i64, _vp]),
    "moe_expert_ffn_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "moe_expert_ffn_workspace_layout": (_i32, [_i32, _i32, _i32, _i32, _i32, ctypes.POINTER(_sz),
                                               ctypes.POINTER(_sz)]),
    "moe_expert_ffn": (_i32, [_i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _u32,
                              _vp, _vp, _sz, _vp]),
    "moe_expert_ffn_noalloc": (_i32, [_i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _i32, _u32,
                                      _vp, _vp]),
    "moe_expert_ffn_rmsnorm": (_i32, [_i32, _vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, ctypes.c_float, _vp, _vp,
                                      _vp, _i32, _u32, _vp, _vp, _sz, _vp]),
    "qg_hbm_read_probe": (_i32, [_vp, _sz, _vp, _vp]),
    "qg_strerror": (_cp, [_i32]),
    "qg_last_error": (_cp, []),
    "qg_version": (_cp, []),
}
EXPORTED_SYMBOLS = tuple(_SIGNATURES)


class QGLibraryMissing(RuntimeError):
    """libqgemv.so has not been built; there is no fallback."""


class QGError(RuntimeError):
    def __init__(self, code: int, func: str, detail: str):
        self.code = code
        self.func = func
        self.detail = detail
        super().__init__(f"{func} failed with {code} ({_strerror(code)}): {detail}")


def lib_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load():
    """Load (once) and return the ctypes handle of libqgemv.so."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            path = lib_path()
            if not os.path.exists(path):
                raise QGLibraryMissing(f"{path} is missing; build it with "
                                       "`python -m block_quantized_decode_qgemv_amd.build`")
            lib = ctypes.CDLL(path)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
    return _lib


def _strerror(code: int) -> str:
    try:
        return load().qg_strerror(code).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return "?"


def _check(rc: int, func: str) -> None:
    if rc != 0:
        raise QGError(rc, func, load().qg_last_error().decode())


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        return FORMATS[fmt.lower()]
    return int(fmt)


def _dev(t, dtype=None, name="tensor", nbytes=None):
    """Device pointer of a torch CUDA tensor (checked) or a raw int pointer.

    For a tensor, `nbytes` is the size the call reads or writes through it: a
    smaller tensor raises ValueError here, before anything is launched.  A raw
    int pointer is passed through unchecked (the caller vouches for it)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not getattr(t, "is_cuda", False):
        raise TypeError(f"{name} must be a device (cuda/hip) tensor or an int device pointer")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if nbytes is not None:
        have = t.numel() * t.element_size()
        if have < nbytes:
            raise ValueError(f"{name} holds {have} bytes; the call needs {nbytes}")
    return t.data_ptr()


def _packed_bytes(fmt, n, k) -> int:
    """Bytes of a packed [n][k] matrix, or 0 for arguments the library rejects
    (it then reports the error itself)."""
    return qg_packed_size(fmt, n, k) if n > 0 and k > 0 else 0


def _ws(ws, ws_bytes, name="ws"):
    return _dev(ws, None, name, ws_bytes if ws_bytes > 0 else None)


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _torch_dtypes():
    import torch

    return torch.float32, torch.uint8


# -------------------------------------------------------------------- sizes

def qg_packed_size(fmt, n: int, k: int) -> int:
    return load().qg_packed_size(_fmt(fmt), n, k)


def qg_codes_plane_size(fmt, n: int, k: int) -> int:
    return load().qg_codes_plane_size(_fmt(fmt), n, k)


def qg_codes_plane_offset(fmt, n: int, k: int) -> int:
    """Where the codes plane ends and the meta plane begins (see qgemv.h)."""
    return load().qg_codes_plane_offset(_fmt(fmt), n, k)


def qg_block_size(fmt) -> int:
    return load().qg_block_size(_fmt(fmt))


def qgemv_workspace_size(fmt, n: int, k: int, b: int = 1) -> int:
    return load().qgemv_workspace_size(_fmt(fmt), n, k, b)


def moe_expert_ffn_workspace_size(t: int, e: int, h: int, i: int, top_k: int) -> int:
    return load().moe_expert_ffn_workspace_size(t, e, h, i, top_k)


def moe_expert_ffn_workspace_layout(t: int, e: int, h: int, i: int, top_k: int) -> tuple[int, int]:
    """(hsel byte offset, h byte offset) of a finished MoE call's workspace
    (see moe_expert_ffn_workspace_layout in qgemv.h)."""
    hs, ho = _sz(0), _sz(0)
    _check(load().moe_expert_ffn_workspace_layout(t, e, h, i, top_k, ctypes.byref(hs), ctypes.byref(ho)),
           "moe_expert_ffn_workspace_layout")
    return hs.value, ho.value


def qg_hbm_read_probe(buf, nbytes: int, sink, stream=None) -> None:
    """Stream-read nbytes of a device buffer (see qg_hbm_read_probe in qgemv.h)."""
    rc = load().qg_hbm_read_probe(_dev(buf, None, "buf", nbytes), nbytes, _dev(sink, None, "sink", 4),
                                  _stream(stream))
    _check(rc, "qg_hbm_read_probe")


def qg_strerror(code: int) -> str:
    return load().qg_strerror(code).decode()


def qg_last_error() -> str:
    return load().qg_last_error().decode()


def qg_version() -> str:
    return load().qg_version().decode()


# --------------------------------------------------------------------- GEMV

def qgemv(fmt, w, x, y, n: int, k: int, b: int = 1, ws=None, ws_bytes: int = 0, stream=None) -> None:
    """y[b][n] = sum_k W[n][k] x[b][k] on the device (see qgemv in qgemv.h)."""
    f32, u8 = _torch_dtypes()
    f, bb = _fmt(fmt), max(b, 0)
    rc = load().qgemv(f, _dev(w, u8, "w", _packed_bytes(f, n, k)), _dev(x, f32, "x", 4 * bb * k),
                      _dev(y, f32, "y", 4 * bb * n), n, k, b, _ws(ws, ws_bytes), ws_bytes, _stream(stream))
    _check(rc, "qgemv")


def _named(cname, fmt):
    def fn(w, x, y, n, k, b=1, ws=None, ws_bytes=0, stream=None):
        f32, u8 = _torch_dtypes()
        bb = max(b, 0)
        rc = getattr(load(), cname)(_dev(w, u8, "w", _packed_bytes(fmt, n, k)), _dev(x, f32, "x", 4 * bb * k),
                                    _dev(y, f32, "y", 4 * bb * n), n, k, b, _ws(ws, ws_bytes), ws_bytes,
                                    _stream(stream))
        _check(rc, cname)

    fn.__name__ = cname
    fn.__doc__ = f"qgemv with the {fmt} format (see {cname} in qgemv.h)."
    return fn


qgemv_q8_0 = _named("qgemv_q8_0", "q8_0")
qgemv_q4_0 = _named("qgemv_q4_0", "q4_0")
qgemv_q4_1 = _named("qgemv_q4_1", "q4_1")
qgemv_q4k = _named("qgemv_q4k", "q4_k")
qgemv_q2k = _named("qgemv_q2k", "q2_k")
qgemv_tern = _named("qgemv_tern", "tern")
qgemv_bin = _named("qgemv_bin", "bin")
qgemv_bin8 = _named("qgemv_bin8", "bin8")
qgemv_tern3 = _named("qgemv_tern3", "tern3")


def qgemv_rmsnorm(fmt, w, x, gamma, eps: float, y, n: int, k: int, b: int = 1, stream=None) -> None:
    """y[b] = W rmsnorm(x[b]; gamma, eps) on the device (see qgemv_rmsnorm in qgemv.h);
    gamma=None means unit gain (gamma folded into the weights)."""
    f32, u8 = _torch_dtypes()
    f, bb = _fmt(fmt), max(b, 0)
    rc = load().qgemv_rmsnorm(f, _dev(w, u8, "w", _packed_bytes(f, n, k)), _dev(x, f32, "x", 4 * bb * k),
                              _dev(gamma, f32, "gamma", 4 * max(k, 0)), float(eps), _dev(y, f32, "y", 4 * bb * n),
                              n, k, b, _stream(stream))
    _check(rc, "qgemv_rmsnorm")


def qquant_device(fmt, w, out, n: int, k: int, status, stream=None) -> None:
    """Quantize fp32 device weights into packed device bytes (see qquant_device
    in qgemv.h); `status` (a device int32) reports device-side failures."""
    f32, u8 = _torch_dtypes()
    f = _fmt(fmt)
    rc = load().qquant_device(f, _dev(w, f32, "w", 4 * max(n, 0) * max(k, 0)), n, k,
                              _dev(out, u8, "out", _packed_bytes(f, n, k)), _dev(status, None, "status", 4),
                              _stream(stream))
    _check(rc, "qquant_device")


def qrequant_workspace_size(n: int, k: int) -> int:
    return load().qrequant_workspace_size(n, k)


def qrequant(src_fmt, src, dst_fmt, dst, n: int, k: int, workspace, ws_bytes: int, status, stream=None) -> None:
    """Decode src and quantize it to dst_fmt on the device (see qrequant in qgemv.h)."""
    _, u8 = _torch_dtypes()
    sf, df = _fmt(src_fmt), _fmt(dst_fmt)
    rc = load().qrequant(sf, _dev(src, u8, "src", _packed_bytes(sf, n, k)), df,
                         _dev(dst, u8, "dst", _packed_bytes(df, n, k)), n, k, _ws(workspace, ws_bytes, "workspace"),
                         ws_bytes, _dev(status, None, "status", 4), _stream(stream))
    _check(rc, "qrequant")


def qg_dequant(fmt, w, out, n: int, k: int, stream=None) -> None:
    f32, u8 = _torch_dtypes()
    f = _fmt(fmt)
    rc = load().qg_dequant(f, _dev(w, u8, "w", _packed_bytes(f, n, k)), _dev(out, f32, "out", 4 * max(n, 0) * max(k, 0)),
                           n, k, _stream(stream))
    _check(rc, "qg_dequant")


# ---------------------------------------------------- host quantizer/packers

def qquant(fmt, w_host, n_threads: int | None = None) -> np.ndarray:
    """fp32 [N, K] host array -> packed uint8 host array (see qquant in qgemv.h)."""
    w = np.ascontiguousarray(w_host, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("w_host must be 2-D [N, K]")
    n, k = w.shape
    size = qg_packed_size(fmt, n, k)
    out = np.empty(max(size, 1), dtype=np.uint8)
    threads = n_threads if n_threads is not None else min(16, os.cpu_count() or 1)
    rc = load().qquant(_fmt(fmt), w.ctypes.data, n, k, out.ctypes.data, threads)
    _check(rc, "qquant")
    return out[:size]


def _codes_and_scales(codes, scale_bits, dtype, name, group=128, block=128):
    """2-D [N, K] codes and fp16 scale bits of shape [N, K/group], checked so
    the host packer never reads past either array (K a multiple of block)."""
    c = np.ascontiguousarray(codes, dtype=dtype)
    s = np.ascontiguousarray(scale_bits, dtype=np.uint16)
    if c.ndim != 2:
        raise ValueError(f"{name}: codes must be 2-D [N, K], got shape {c.shape}")
    n, k = c.shape
    if k % block:
        raise ValueError(f"{name}: K={k} must be a multiple of {block}")
    if s.shape != (n, k // group):
        raise ValueError(f"{name}: scale_bits must have shape {(n, k // group)}, got {s.shape}")
    return c, s, n, k


def qpack_tern(codes, scale_bits) -> np.ndarray:
    t, s, n, k = _codes_and_scales(codes, scale_bits, np.int8, "qpack_tern")
    size = qg_packed_size("tern", n, k)
    out = np.empty(max(size, 1), dtype=np.uint8)
    _check(load().qpack_tern(t.ctypes.data, s.ctypes.data, n, k, out.ctypes.data), "qpack_tern")
    return out[:size]


def qpack_bin(bits, scale_bits) -> np.ndarray:
    bb, s, n, k = _codes_and_scales(bits, scale_bits, np.uint8, "qpack_bin")
    size = qg_packed_size("bin", n, k)
    out = np.empty(max(size, 1), dtype=np.uint8)
    _check(load().qpack_bin(bb.ctypes.data, s.ctypes.data, n, k, out.ctypes.data), "qpack_bin")
    return out[:size]


def qpack_tern3(codes, scale_bits) -> np.ndarray:
    """Ternary codes and fp16 scales per 64 weights -> packed tern3 bytes (see qpack_tern3 in qgemv.h)."""
    t, s, n, k = _codes_and_scales(codes, scale_bits, np.int8, "qpack_tern3", group=64, block=256)
    size = qg_packed_size("tern3", n, k)
    out = np.empty(max(size, 1), dtype=np.uint8)
    _check(load().qpack_tern3(t.ctypes.data, s.ctypes.data, n, k, out.ctypes.data), "qpack_tern3")
    return out[:size]


def qpack_bin8(bits, scale_bits) -> np.ndarray:
    """1-bit codes and fp16 block scales -> packed bin8 bytes (see qpack_bin8 in qgemv.h)."""
    bb, s, n, k = _codes_and_scales(bits, scale_bits, np.uint8, "qpack_bin8")
    size = qg_packed_size("bin8", n, k)
    out = np.empty(max(size, 1), dtype=np.uint8)
    _check(load().qpack_bin8(bb.ctypes.data, s.ctypes.data, n, k, out.ctypes.data), "qpack_bin8")
    return out[:size]


# ---------------------------------------------------------------- MoE layer

def _moe_sizes(fmt, e, h, i, t):
    """Bytes each MoE argument spans: (gate/up, down, activations, logits, shared logits)."""
    f = _fmt(fmt)
    ok = e > 0 and h > 0 and i > 0 and t > 0
    gu = (e + 1) * _packed_bytes(f, 2 * i, h) if ok else 0
    dn = (e + 1) * _packed_bytes(f, h, i) if ok else 0
    return f, gu, dn, 4 * max(t, 0) * max(h, 0), 4 * max(t, 0) * max(e, 0), 4 * max(t, 0)


def moe_expert_ffn(fmt, w_gate_up, w_down, e: int, h: int, i: int, top_k: int, x, residual,
                   router_logits, shared_gate_logit, t: int, out, workspace, ws_bytes: int,
                   flags: int = 0, stream=None) -> None:
    """Routed expert layer (see moe_expert_ffn in qgemv.h)."""
    f32, u8 = _torch_dtypes()
    f, gu, dn, act, lg, sl = _moe_sizes(fmt, e, h, i, t)
    rc = load().moe_expert_ffn(f, _dev(w_gate_up, u8, "w_gate_up", gu), _dev(w_down, u8, "w_down", dn),
                               e, h, i, top_k, _dev(x, f32, "x", act), _dev(residual, f32, "residual", act),
                               _dev(router_logits, f32, "router_logits", lg),
                               _dev(shared_gate_logit, f32, "shared_gate_logit", sl), t, flags,
                               _dev(out, f32, "out", act), _ws(workspace, ws_bytes, "workspace"), ws_bytes,
                               _stream(stream))
    _check(rc, "moe_expert_ffn")


def moe_expert_ffn_noalloc(fmt, w_gate_up, w_down, e: int, h: int, i: int, top_k: int, x, residual,
                           router_logits, shared_gate_logit, t: int, out, flags: int = 0, stream=None) -> None:
    """Routed expert layer with the library's own device scratch as its
    workspace: no allocation (see moe_expert_ffn_noalloc in qgemv.h)."""
    f32, u8 = _torch_dtypes()
    f, gu, dn, act, lg, sl = _moe_sizes(fmt, e, h, i, t)
    rc = load().moe_expert_ffn_noalloc(f, _dev(w_gate_up, u8, "w_gate_up", gu), _dev(w_down, u8, "w_down", dn),
                                       e, h, i, top_k, _dev(x, f32, "x", act), _dev(residual, f32, "residual", act),
                                       _dev(router_logits, f32, "router_logits", lg),
                                       _dev(shared_gate_logit, f32, "shared_gate_logit", sl), t, flags,
                                       _dev(out, f32, "out", act), _stream(stream))
    _check(rc, "moe_expert_ffn_noalloc")


def moe_expert_ffn_rmsnorm(fmt, w_gate_up, w_down, e: int, h: int, i: int, top_k: int, x, gamma, eps: float,
                           residual, router_logits, shared_gate_logit, t: int, out, workspace, ws_bytes: int,
                           flags: int = 0, stream=None) -> None:
    """Routed expert layer on RMS-normalised x (see moe_expert_ffn_rmsnorm in qgemv.h);
    gamma=None means unit gain (the gain folded into the gate/up weights)."""
    f32, u8 = _torch_dtypes()
    f, gu, dn, act, lg, sl = _moe_sizes(fmt, e, h, i, t)
    rc = load().moe_expert_ffn_rmsnorm(f, _dev(w_gate_up, u8, "w_gate_up", gu), _dev(w_down, u8, "w_down", dn),
                                       e, h, i, top_k, _dev(x, f32, "x", act), _dev(gamma, f32, "gamma", 4 * max(h, 0)),
                                       float(eps), _dev(residual, f32, "residual", act),
                                       _dev(router_logits, f32, "router_logits", lg),
                                       _dev(shared_gate_logit, f32, "shared_gate_logit", sl), t, flags,
                                       _dev(out, f32, "out", act), _ws(workspace, ws_bytes, "workspace"), ws_bytes,
                                       _stream(stream))
    _check(rc, "moe_expert_ffn_rmsnorm")
