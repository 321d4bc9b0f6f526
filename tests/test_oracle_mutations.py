"""Plant plausible mistakes in (copies of) the oracle's arithmetic, on the CPU,
and check that the pins catch each one.  Nothing here touches the GPU path."""
import numpy as np
import pytest

from oracle import page_listing as PL

F32 = np.float32


@pytest.fixture(scope="module")
def page_w():
    return PL.page_weights()


def _printed(golden):
    return {r[0]: float(r[2]) for r in golden("handbook_error_table.txt")}


def _q4_0_unsigned(w):
    b = np.asarray(w, F32).reshape(-1, 32)
    d = PL._div(np.abs(b).max(axis=1, keepdims=True), F32(8))   # mistake: |max| / 8
    return (np.clip(np.rint(PL._div(b, d)), -8, 7) * d).reshape(-1), 4.5


def _q4_0_sign_flip(w):
    b = np.asarray(w, F32).reshape(-1, 32)
    j = np.argmax(np.abs(b), axis=1)[:, None]
    d = PL._div(np.take_along_axis(b, j, axis=1), F32(8))        # mistake: / +8
    return (np.clip(np.rint(PL._div(b, d)), -8, 7) * d).reshape(-1), 4.5


def _q4_1_sixteen(w):
    b = np.asarray(w, F32).reshape(-1, 32)
    lo, hi = b.min(axis=1, keepdims=True), b.max(axis=1, keepdims=True)
    d = PL._div(hi - lo, F32(16))                                # mistake: 16 levels
    return (np.clip(np.rint(PL._div(b - lo, d)), 0, 15) * d + lo).reshape(-1), 5.0


def _q4_k_no_min_clamp(w):
    b = np.asarray(w, F32).reshape(-1, 8, 32)
    lo = b.min(axis=2, keepdims=True)                            # mistake: no clamp(max=0)
    hi = b.max(axis=2, keepdims=True)
    sc, mn = PL._div(hi - lo, F32(15)), -lo
    dsc = PL._div(sc.max(axis=1, keepdims=True), F32(63))
    dmn = PL._div(np.abs(mn).max(axis=1, keepdims=True), F32(63))
    sc_q = np.clip(np.rint(PL._div(sc, dsc)), 1, 63) * dsc
    mn_q = np.clip(np.rint(PL._div(mn, dmn)), 0, 63) * dmn
    q = np.clip(np.rint(PL._div(b + mn_q, sc_q)), 0, 15)
    return (q * sc_q - mn_q).reshape(-1), 4.5


def _q4_k_scale_bits_5(w):
    b = np.asarray(w, F32).reshape(-1, 8, 32)
    lo = np.minimum(b.min(axis=2, keepdims=True), F32(0))
    hi = b.max(axis=2, keepdims=True)
    sc, mn = PL._div(hi - lo, F32(15)), -lo
    dsc = PL._div(sc.max(axis=1, keepdims=True), F32(31))        # mistake: 5-bit scale codes
    dmn = PL._div(mn.max(axis=1, keepdims=True), F32(31))
    sc_q = np.clip(np.rint(PL._div(sc, dsc)), 1, 31) * dsc
    mn_q = np.clip(np.rint(PL._div(mn, dmn)), 0, 31) * dmn
    q = np.clip(np.rint(PL._div(b + mn_q, sc_q)), 0, 15)
    return (q * sc_q - mn_q).reshape(-1), 4.5


def _q8_0_128(w):
    b = np.asarray(w, F32).reshape(-1, 32)
    d = PL._div(np.abs(b).max(axis=1, keepdims=True), F32(128))   # mistake: / 128
    return (np.clip(np.rint(PL._div(b, d)), -127, 127) * d).reshape(-1), 8.5


@pytest.mark.parametrize("name,fn", [
    ("Q4_0", _q4_0_unsigned), ("Q4_0", _q4_0_sign_flip), ("Q4_1", _q4_1_sixteen),
    ("Q4_K", _q4_k_scale_bits_5), ("Q8_0", _q8_0_128),
])
def test_planted_mistake_breaks_error_table(page_w, golden, name, fn):
    deq, _ = fn(page_w)
    assert round(PL.relative_error(deq, page_w), 4) != _printed(golden)[name]


def test_planted_missing_min_clamp_breaks_handbuilt_roundtrip():
    """Student-t blocks always have a negative minimum, so the table cannot see
    a missing min clamp; the hand-built all-positive sub-block does."""
    from oracle import formats as F
    from tests.test_oracle_formats import _handbuilt_kquant

    blk = _handbuilt_kquant(15)
    w = F.dequant("q4_k", blk)
    deq, _ = _q4_k_no_min_clamp(w.reshape(-1))
    assert not np.array_equal(deq.reshape(w.shape), w)
    deq_ok, _ = PL.q4_k(w.reshape(-1))
    np.testing.assert_array_equal(deq_ok.reshape(w.shape), w)
