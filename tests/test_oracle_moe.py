"""Oracle pins for the routed MoE layer (CPU only)."""
import numpy as np
import pytest

import workloads
from oracle import formats as F
from oracle import moe as M
from tests import oracle_pins as P


def _experts(e, h, i, seed=0, identical=False):
    wg, wu, wd = [], [], []
    for ex in range(e + 1):
        tid = 0 if identical else ex
        wg.append(F.dequant("q4_k", F.quantize("q4_k", workloads.student_t_weights(i, h, seed, 3 * tid))))
        wu.append(F.dequant("q4_k", F.quantize("q4_k", workloads.student_t_weights(i, h, seed, 3 * tid + 1))))
        wd.append(F.dequant("q4_k", F.quantize("q4_k", workloads.student_t_weights(h, i, seed, 3 * tid + 2))))
    return wg, wu, wd


def test_softmax_and_route_basics():
    logits = workloads.normal((4, 16), 1)
    ids, w, p = M.route(logits, 4)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-15)
    for t in range(4):
        assert list(ids[t]) == M.top_k_bruteforce(p[t], 4)
        assert np.all(np.diff(w[t]) <= 0)
        # top-K by probability is top-K by logit (softmax is monotone)
        assert set(ids[t]) == set(np.argsort(-logits[t], kind="stable")[:4])
    ids_r, w_r, _ = M.route(logits, 4, renorm=True)
    np.testing.assert_array_equal(ids_r, ids)
    np.testing.assert_allclose(w_r.sum(axis=1), 1.0, rtol=1e-15)


def test_route_ties_prefer_lower_index():
    logits = np.zeros((1, 8), np.float32)
    logits[0, [6, 2, 5]] = 1.0
    ids, _, _ = M.route(logits, 4)
    assert list(ids[0]) == [2, 5, 6, 0]


def test_route_nan_counts_as_minus_inf_and_signed_zeros_tie():
    """NaN logits route like -inf (the stated reading); -0 and +0 are equal
    logits, so the lower index wins between them; -inf experts still fill the
    top-K after every finite one, lower index first, with weight 0."""
    logits = np.array([[np.nan, -1.0, np.nan, 2.0, -1.0, 0.5],
                       [-0.0, -1.0, 0.0, -0.0, -2.0, -3.0],
                       [-np.inf, 0.3, -np.inf, 0.3, -np.inf, -np.inf]], np.float32)
    ids, w, _ = M.route(logits, 4)
    assert list(ids[0]) == [3, 5, 1, 4]
    assert list(ids[1]) == [0, 2, 3, 1]
    assert list(ids[2]) == [1, 3, 0, 2]
    assert w[2, 2] == 0.0 and w[2, 3] == 0.0
    nan_free = np.where(np.isnan(logits), -np.inf, logits)
    ids2, w2, _ = M.route(nan_free, 4)
    np.testing.assert_array_equal(ids, ids2)
    np.testing.assert_array_equal(w, w2)


def test_identical_experts_closed_form():
    e, h, i, t = 6, 256, 256, 3
    wg, wu, wd = _experts(e, h, i, identical=True)
    x = workloads.normal((t, h), 2)
    res = workloads.normal((t, h), 2, 1)
    logits = workloads.normal((t, e), 2, 2)
    s = workloads.normal((t,), 2, 3)
    ref = M.moe_ref(wg, wu, wd, x, res, logits, s, 2)
    _, _, _, o = M.expert_forward(wg[0], wu[0], wd[0], x)
    want = res.astype(np.float64) + (ref["weights"].sum(axis=1) + M.sigmoid(s))[:, None] * o
    np.testing.assert_allclose(ref["out"], want, rtol=1e-12, atol=1e-12)


def test_shared_gate_off_and_dominant_logit():
    e, h, i = 5, 256, 256
    wg, wu, wd = _experts(e, h, i, seed=1)
    x = workloads.normal((1, h), 3)
    res = np.zeros((1, h), np.float32)
    logits = np.full((1, e), -30.0, np.float32)
    logits[0, 3] = 30.0
    ref = M.moe_ref(wg, wu, wd, x, res, logits, np.array([-np.inf], np.float32), 1)
    assert ref["ids"][0, 0] == 3 and ref["sigma"][0] == 0.0
    _, _, _, o3 = M.expert_forward(wg[3], wu[3], wd[3], x)
    np.testing.assert_allclose(ref["out"], ref["weights"][0, 0] * o3, rtol=1e-12)
    assert ref["weights"][0, 0] == pytest.approx(1.0, abs=1e-20)


def test_silu_and_sigmoid_values():
    assert M.silu(0.0) == 0.0
    assert M.silu(1.0) == pytest.approx(1.0 / (1.0 + np.exp(-1.0)))
    assert M.sigmoid(0.0) == 0.5
    assert M.silu(-50.0) == pytest.approx(0.0, abs=1e-18)


def test_tolerance_is_positive_and_finite():
    e, h, i, t = 3, 256, 256, 2
    wg, wu, wd = _experts(e, h, i, seed=2)
    x = workloads.normal((t, h), 4)
    res = workloads.normal((t, h), 4, 1)
    logits = workloads.normal((t, e), 4, 2)
    s = workloads.normal((t,), 4, 3)
    ref = M.moe_ref(wg, wu, wd, x, res, logits, s, 2)
    tol = M.out_tolerance(wg, wu, wd, x, res, ref)
    assert np.all(np.isfinite(tol)) and np.all(tol > 0)
    assert np.all(tol < 1e-3 * (np.abs(ref["out"]) + 1))


def test_interleave_gate_up():
    a = np.arange(6).reshape(3, 2)
    b = -np.arange(6).reshape(3, 2)
    il = M.interleave_gate_up(a, b)
    np.testing.assert_array_equal(il[0::2], a)
    np.testing.assert_array_equal(il[1::2], b)


# ----------------------------------------------------------------------------
# independent pins (tests/oracle_pins.py): brute force with math.fsum


def test_expert_forward_against_fsum():
    """expert_forward against a brute-force expert (H != I and square)."""
    P.expert_forward_fsum(M)


def test_route_against_fsum():
    P.route_pin(M)


def test_moe_ref_against_fsum():
    """The whole layer -- route, experts, gated combine and residual -- by
    brute force on tiny experts."""
    P.moe_combine_fsum(M)
