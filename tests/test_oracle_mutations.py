"""Planted mistakes in the oracle's own source, each rejected by a pin.

Every case below edits the source of ``oracle.formats`` or ``oracle.moe``
(tests/mutate.py builds the edited module; the oracle on disk is untouched)
and runs the pin named next to it from tests/oracle_pins.py, which must fail
on the mutant.  The same pins pass on the oracle itself (test_oracle_formats,
test_oracle_moe).  CPU only.
"""
import numpy as np
import pytest

from oracle import formats as OF
from oracle import moe as OM
from oracle import page_sample
from tests import oracle_pins as P
from tests.mutate import mutant


@pytest.fixture(scope="module")
def page_w():
    return page_sample.page_weights()


@pytest.fixture(scope="module")
def printed():
    from tests.conftest import read_golden

    return {r[0]: float(r[2]) for r in read_golden("handbook_error_table.txt")}


KQ_5BIT = [
    ("_div(sc.max(axis=2), F32(63))", "_div(sc.max(axis=2), F32(31))"),
    ("_div(mn.max(axis=2), F32(63))", "_div(mn.max(axis=2), F32(31))"),
    ("np.clip(np.rint(_div(sc, dd)), 1, 63)", "np.clip(np.rint(_div(sc, dd)), 1, 31)"),
    ("np.clip(np.rint(_div(mn, dm)), 0, 63)", "np.clip(np.rint(_div(mn, dm)), 0, 31)"),
]

# (name, edits, pin) -- pin is called with the mutant module and must fail
FORMAT_MUTANTS = [
    ("q8_0 divides by 128", [("_div(a, F32(127))", "_div(a, F32(128))")], "table"),
    ("q4_0 scale divided by +8", [("_div(bj, F32(-8))", "_div(bj, F32(8))")], "table"),
    ("q4_0 unsigned scale |max| / 8", [("_div(bj, F32(-8))", "_div(np.abs(bj), F32(8))")], "table"),
    ("q4_0 tie takes the last index",
     [("j = np.argmax(np.abs(b), axis=2)", "j = b.shape[2] - 1 - np.argmax(np.abs(b)[..., ::-1], axis=2)")],
     "q4_0_tie"),
    ("q4_1 sixteen levels", [("_div(hi - lo, F32(15))", "_div(hi - lo, F32(16))")], "table"),
    ("q4_1 offset from the max", [("m_st = _store(lo, literal)", "m_st = _store(hi, literal)")], "table"),
    ("k-quant 5-bit scale codes", KQ_5BIT, "table"),
    ("k-quant codes floored", [("np.clip(np.rint(_div(b + Mn, S)), 0, qmax)",
                                "np.clip(np.floor(_div(b + Mn, S)), 0, qmax)")], "table"),
    ("k-quant minimum not clamped to <= 0", [("lo = np.minimum(b.min(axis=3), F32(0))", "lo = b.min(axis=3)")],
     "kquant_roundtrip"),
    ("codes against the unrounded scale (R1)",
     [("d = scale_values(d_st)[..., None]\n    q = np.where(d == 0, F32(0), np.clip(np.rint(_div(b, d)), -127, 127))",
       "d = _div(a, F32(127))[..., None]\n    q = np.where(d == 0, F32(0), np.clip(np.rint(_div(b, d)), -127, 127))")],
     "q8_0_r1"),
    ("q4_1 decode subtracts m", [("return nn.astype(F32) * d + m", "return nn.astype(F32) * d - m")], "q4_1_roundtrip"),
    ("nibbles high first", [("(v[:, 0::2] | (v[:, 1::2] << 4))", "((v[:, 0::2] << 4) | v[:, 1::2])")], "bytes"),
    ("k-quant pair holds t low, s high",
     [('p = blk["s"].astype(np.uint32) | (blk["t"].astype(np.uint32) << 6)',
       'p = blk["t"].astype(np.uint32) | (blk["s"].astype(np.uint32) << 6)')], "kquant_meta"),
    ("rows not interleaved", [(".reshape(ng, units, UNIT).transpose(1, 0, 2).reshape(-1)",
                               ".reshape(ng, units, UNIT).reshape(-1)")], "interleave"),
    ("bin bit 1 means -1",
     [('return (2 * bb.astype(np.int16) - 1).astype(F32) * _per_block(scale_values(blk["d"]), 128, bb.shape[1])',
       'return (1 - 2 * bb.astype(np.int16)).astype(F32) * _per_block(scale_values(blk["d"]), 128, bb.shape[1])')],
     "tern_bin"),
    ("tern field offset 2", [("(f.astype(np.int16) - 1)", "(f.astype(np.int16) - 2)")], "tern_bin"),
    ("bin8 step over 256", [("/ F32(255)).astype(F32)", "/ F32(256)).astype(F32)")], "bin8"),
    ("bin8 codes floored", [("np.clip(np.rint((d - base[:, None]) / step[:, None]), 0, 255)",
                             "np.clip(np.floor((d - base[:, None]) / step[:, None]), 0, 255)")], "bin8"),
    ("bin8 base from the max", [("base = d.min(axis=1)", "base = d.max(axis=1)")], "bin8"),
    ("tern3 digits most significant first",
     [("main[..., l] * 3 ** l for l in range(5)", "main[..., l] * 3 ** (4 - l) for l in range(5)")], "tern3"),
    ("tern3 digits of a byte four columns apart",
     [("main = g[..., :60].reshape(n, nb, 4, 12, 5)",
       "main = g[..., :60].reshape(n, nb, 4, 3, 5, 4).swapaxes(-1, -2).reshape(n, nb, 4, 12, 5)")], "tern3"),
    ("tern3 tail field transposed",
     [("field = sum(tail[:, :, s, :] << (2 * s) for s in range(4))",
       "field = sum(tail[:, :, :, s] << (2 * s) for s in range(4))")], "tern3"),
    ("tern3 field offset 0", [("(f.astype(F32) - F32(1))", "f.astype(F32)")], "tern3"),
    ("tern3 scales after the field",
     [("meta = np.concatenate([scales, field.astype(np.uint8)], axis=-1)",
       "meta = np.concatenate([field.astype(np.uint8), scales], axis=-1)")], "tern3"),
]

MOE_MUTANTS = [
    ("SwiGLU on the up projection", [("    u = _gemv64(wu, x)\n    h = silu(g) * u\n",
                                      "    u = _gemv64(wu, x)\n    h = g * silu(u)\n")], "expert"),
    ("down projection transposed",
     [("o = np.asarray(h, np.float64) @ np.asarray(wd, np.float32).astype(np.float64).T",
       "o = np.asarray(h, np.float64) @ np.asarray(wd, np.float32).astype(np.float64)")], "expert"),
    ("silu replaced by sigmoid", [("return z / (1.0 + np.exp(-z))", "return 1.0 / (1.0 + np.exp(-z))")], "expert"),
    ("top-K always renormalised", [("    if renorm:\n        w = w / w.sum", "    if True:\n        w = w / w.sum")],
     "route"),
    ("ties to the higher index", [('order = np.argsort(-p[i], kind="stable")',
                                   'order = len(p[i]) - 1 - np.argsort(-p[i][::-1], kind="stable")')], "route"),
    ("softmax not normalised", [("return e / e.sum(axis=-1, keepdims=True)", "return e")], "route"),
    ("shared expert ungated", [("out[i] += sig[i] * o_all[i, top_k]", "out[i] += o_all[i, top_k]")], "combine"),
    ("residual dropped", [('out = np.asarray(residual, np.float32).astype(np.float64).copy()',
                           'out = np.zeros_like(np.asarray(residual, np.float32), dtype=np.float64)')], "combine"),
]


def _run_format_pin(kind, mod, page_w, printed):
    if kind == "table":
        P.error_table_literal(mod, page_w, printed)
    elif kind == "q4_0_tie":
        P.q4_0_tie_takes_first_index(mod)
    elif kind == "kquant_roundtrip":
        P.roundtrip_kquant(mod, "q4_k", 15)
    elif kind == "q8_0_r1":
        P.q8_0_codes_against_stored_scale(mod)
    elif kind == "q4_1_roundtrip":
        P.roundtrip_q4_1(mod)
    elif kind == "bytes":
        P.byte_order(mod)
    elif kind == "kquant_meta":
        P.kquant_meta_bytes(mod)
    elif kind == "interleave":
        P.row_interleave(mod)
    elif kind == "tern_bin":
        P.roundtrip_tern_bin(mod)
    elif kind == "bin8":
        P.bin8_affine_exact(mod)
        P.bin8_rounding_bound(mod)
    elif kind == "tern3":
        P.tern3_bytes(mod)
    else:
        raise KeyError(kind)


def _run_moe_pin(kind, mod):
    {"expert": P.expert_forward_fsum, "route": P.route_pin, "combine": P.moe_combine_fsum}[kind](mod)


@pytest.mark.parametrize("name,edits,pin", FORMAT_MUTANTS, ids=[m[0] for m in FORMAT_MUTANTS])
def test_format_mutant_rejected(page_w, printed, name, edits, pin):
    _run_format_pin(pin, OF, page_w, printed)  # the pin holds on the oracle itself
    mod = mutant(OF, edits)
    with pytest.raises((AssertionError, ValueError, IndexError)):
        _run_format_pin(pin, mod, page_w, printed)


@pytest.mark.parametrize("name,edits,pin", MOE_MUTANTS, ids=[m[0] for m in MOE_MUTANTS])
def test_moe_mutant_rejected(name, edits, pin):
    _run_moe_pin(pin, OM)
    mod = mutant(OM, edits)
    with pytest.raises((AssertionError, ValueError)):
        _run_moe_pin(pin, mod)


def test_transposed_down_on_square_expert_fails_on_values():
    """On the square expert the transposed down projection runs and must fail
    on the values, not on a shape error."""
    mod = mutant(OM, [("o = np.asarray(h, np.float64) @ np.asarray(wd, np.float32).astype(np.float64).T",
                       "o = np.asarray(h, np.float64) @ np.asarray(wd, np.float32).astype(np.float64)")])
    wg, wu, wd, x = P._tiny_expert(128, 128, 12)
    _, _, _, o = mod.expert_forward(wg, wu, wd, x)
    eo = P.expert_fsum(wg, wu, wd, x[0])[3]
    assert not np.allclose(o[0], eo, rtol=1e-6)
