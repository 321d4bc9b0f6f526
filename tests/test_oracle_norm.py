"""Pins of the RMS-norm + GEMV oracle (oracle/norm.py) against what the
definition fixes, and planted mistakes (in copies, on the CPU) that the pins
must catch.  Nothing here touches the GPU path."""
import math

import numpy as np
import pytest

from oracle import gemv as OG
from oracle import norm as ON

F32 = np.float32


def _w(n, k, seed=0):
    return np.random.default_rng(seed).standard_normal((n, k)).astype(F32)


def _close(a, b, rel=1e-12):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return bool(np.all(np.abs(a - b) <= rel * (np.abs(b) + 1e-300) + 1e-13))


# Each pin takes an implementation of y = W rmsnorm(x; gamma, eps) and says
# whether it agrees with what the definition fixes.

def pin_hand_vectors(impl):
    eye = np.eye(4, dtype=F32)  # W = I exposes xhat itself
    ok = _close(impl(eye, [[3, 4, 0, 0]], np.ones(4, F32), 0.0), [[1.2, 1.6, 0, 0]])          # rms = 2.5
    ok &= _close(impl(eye, [[2, 2, 2, 2]], np.ones(4, F32), 5.0), [[2 / 3] * 4])             # sqrt(4 + 5) = 3
    ok &= _close(impl(eye, [[1, -1, 1, -1]], F32([0.5, 2, 1, -1]), 0.0), [[0.5, -2, 1, 1]])  # rms = 1
    ok &= _close(impl(eye, [[3, 4, 0, 0], [1, 1, 1, 1]], np.ones(4, F32), 0.0),
                 [[1.2, 1.6, 0, 0], [1, 1, 1, 1]])                                            # rows apart
    return ok


def pin_constant_row_sums(impl):
    w = _w(5, 64, 1)
    rows = np.array([math.fsum(map(float, r)) for r in w])
    ok = _close(impl(w, np.full((1, 64), 7.5, F32), np.ones(64, F32), 0.0)[0], rows)
    ok &= _close(impl(w, np.full((1, 64), -0.25, F32), np.ones(64, F32), 0.0)[0], -rows)
    return ok


def pin_zero_vector(impl):
    return bool(np.all(impl(_w(3, 32, 2), np.zeros((1, 32), F32), np.ones(32, F32), 1e-6) == 0.0))


def pin_scale_invariance(impl):
    rng = np.random.default_rng(3)
    w, x, g = _w(6, 96, 4), rng.standard_normal((2, 96)).astype(F32), rng.uniform(0.5, 2, 96).astype(F32)
    return _close(impl(w, x, g, 0.0), impl(w, x * F32(8), g, 0.0), 1e-12)


def pin_unit_mean_square(impl):
    x = np.random.default_rng(5).standard_normal((3, 128)).astype(F32)
    xhat = impl(np.eye(128, dtype=F32), x, np.ones(128, F32), 0.0)
    return _close(np.mean(xhat * xhat, axis=1), np.ones(3))


def pin_plain_gemv_identity(impl):
    rng = np.random.default_rng(6)
    w, x = _w(7, 160, 7), rng.standard_normal((2, 160)).astype(F32)
    g = (2.0 ** rng.integers(-2, 3, 160)).astype(F32)  # x * gamma stays exact in fp32
    eps = 0.125
    r = np.sqrt(np.array([math.fsum(float(v) ** 2 for v in row) for row in x]) / 160 + eps)
    return _close(impl(w, x, g, eps) * r[:, None], OG.gemv_ref(w, x * g), 1e-11)


def pin_brute_force(impl):
    rng = np.random.default_rng(8)
    w, x, g = _w(3, 8, 9), rng.standard_normal((2, 8)).astype(F32), rng.standard_normal(8).astype(F32)
    eps = 0.01
    want = np.empty((2, 3))
    for b in range(2):
        r = math.sqrt(math.fsum(float(v) * float(v) for v in x[b]) / 8 + float(F32(eps)))
        for n in range(3):
            want[b, n] = math.fsum(float(w[n, k]) * float(x[b, k]) * float(g[k]) / r for k in range(8))
    return _close(impl(w, x, g, eps), want, 1e-12)


PINS = [pin_hand_vectors, pin_constant_row_sums, pin_zero_vector, pin_scale_invariance,
        pin_unit_mean_square, pin_plain_gemv_identity, pin_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_meets_pin(pin):
    assert pin(ON.gemv_rmsnorm_ref)


def test_gain_folds_into_the_weights():
    """W rmsnorm(x; gamma) == (W diag(gamma)) rmsnorm(x; 1): the reading that
    gamma scales columns, which is what lets a caller fold it into W."""
    rng = np.random.default_rng(9)
    w, x = _w(5, 64, 11), rng.standard_normal((2, 64)).astype(F32)
    g = (2.0 ** rng.integers(-2, 3, 64)).astype(F32)  # exact column scaling of W
    a = ON.gemv_rmsnorm_ref(w, x, g, 1e-3)
    b = ON.gemv_rmsnorm_ref((w * g[None, :]).astype(F32), x, np.ones(64, F32), 1e-3)
    assert _close(a, b, 1e-12)


def test_rms_pass_alone():
    assert _close(ON.rms([[3, 4, 0, 0]], 0.0), [2.5])
    assert _close(ON.rms([[2, 2, 2, 2]], 5.0), [3.0])
    assert _close(ON.rmsnorm_ref([[3, 4, 0, 0]], np.ones(4, F32), 0.0), [[1.2, 1.6, 0, 0]])


def test_tolerance_scales_with_normalised_terms():
    w = np.eye(4, dtype=F32)
    t = ON.tolerance(w, [[3, 4, 0, 0]], np.ones(4, F32), 0.0)
    assert _close(t, [[ON.REL_TOL * 1.2 + ON.ABS_TOL, ON.REL_TOL * 1.6 + ON.ABS_TOL, ON.ABS_TOL, ON.ABS_TOL]])
    ok, ratio, _ = ON.check([[1.2, 1.6, 0, 0]], w, [[3, 4, 0, 0]], np.ones(4, F32), 0.0)
    assert ok and ratio == 0.0
    ok, _, idx = ON.check([[1.2, 1.6 * (1 + 1e-4), 0, 0]], w, [[3, 4, 0, 0]], np.ones(4, F32), 0.0)
    assert not ok and idx == (0, 1)


# ------------------------------------------------------------ planted mistakes

def _x64(x):
    return np.atleast_2d(np.asarray(x, F32)).astype(np.float64)


def _sum_not_mean(w, x, g, eps):
    x = _x64(x)
    r = np.sqrt(np.sum(x * x, axis=1) + eps)
    return (x * np.asarray(g, np.float64) / r[:, None]) @ np.asarray(w, np.float64).T


def _eps_outside_sqrt(w, x, g, eps):
    x = _x64(x)
    r = np.sqrt(np.mean(x * x, axis=1)) + eps
    return (x * np.asarray(g, np.float64) / r[:, None]) @ np.asarray(w, np.float64).T


def _no_gamma(w, x, g, eps):
    x = _x64(x)
    r = np.sqrt(np.mean(x * x, axis=1) + eps)
    return (x / r[:, None]) @ np.asarray(w, np.float64).T


def _no_sqrt(w, x, g, eps):
    x = _x64(x)
    r = np.mean(x * x, axis=1) + eps
    return (x * np.asarray(g, np.float64) / r[:, None]) @ np.asarray(w, np.float64).T


def _whole_batch(w, x, g, eps):
    x = _x64(x)
    r = np.sqrt(np.mean(x * x) + eps)
    return (x * np.asarray(g, np.float64) / r) @ np.asarray(w, np.float64).T


def _mean_subtracted(w, x, g, eps):  # layer norm's centring where RMS norm has none
    x = _x64(x)
    x = x - x.mean(axis=1, keepdims=True)
    r = np.sqrt(np.mean(x * x, axis=1) + eps)
    return (x * np.asarray(g, np.float64) / r[:, None]) @ np.asarray(w, np.float64).T


@pytest.mark.parametrize("mutant", [_sum_not_mean, _eps_outside_sqrt, _no_gamma, _no_sqrt, _whole_batch,
                                    _mean_subtracted], ids=lambda f: f.__name__)
def test_planted_mistake_fails_a_pin(mutant):
    with np.errstate(all="ignore"):  # centring a constant row divides 0 by 0
        failed = [p.__name__ for p in PINS if not p(mutant)]
    assert failed, f"{mutant.__name__} passes every pin"


# ------------------------------------------------------- norm-fed MoE layer

def _moe_case(t=3, e=6, h=64, i=32, seed=40):
    from oracle import moe as OM

    rng = np.random.default_rng(seed)
    wg = [rng.standard_normal((i, h)).astype(F32) * F32(0.1) for _ in range(e + 1)]
    wu = [rng.standard_normal((i, h)).astype(F32) * F32(0.1) for _ in range(e + 1)]
    wd = [rng.standard_normal((h, i)).astype(F32) * F32(0.1) for _ in range(e + 1)]
    x = rng.standard_normal((t, h)).astype(F32) * F32(3)
    res = rng.standard_normal((t, h)).astype(F32)
    logits = rng.standard_normal((t, e)).astype(F32)
    s = rng.standard_normal(t).astype(F32)
    return OM, wg, wu, wd, x, res, logits, s


def test_moe_norm_reduces_to_moe_on_unit_rms_rows():
    """x of +-1 entries has RMS 1: with gamma = 1 and eps = 0 the norm is the
    identity and the layer equals the (separately pinned) MoE oracle."""
    OM, wg, wu, wd, x, res, logits, s = _moe_case()
    x = np.sign(x).astype(F32)
    got = ON.moe_rmsnorm_ref(wg, wu, wd, x, np.ones(x.shape[1], F32), 0.0, res, logits, s, 2)["out"]
    want = OM.moe_ref(wg, wu, wd, x, res, logits, s, 2)["out"]
    assert _close(got, want, 1e-12)


def test_moe_norm_scale_invariant_and_exact_xhat():
    """Scaling x by 8 (eps = 0) leaves every expert input and so the layer
    unchanged; and the experts see the float64 xhat unrounded (the result
    differs from feeding them xhat rounded to fp32)."""
    OM, wg, wu, wd, x, res, logits, s = _moe_case(seed=41)
    g = (1 + 0.25 * np.random.default_rng(1).standard_normal(x.shape[1])).astype(F32)
    a = ON.moe_rmsnorm_ref(wg, wu, wd, x, g, 0.0, res, logits, s, 3)["out"]
    b = ON.moe_rmsnorm_ref(wg, wu, wd, x * F32(8), g, 0.0, res, logits, s, 3)["out"]
    assert _close(a, b, 1e-12)
    xh = ON.rmsnorm_ref(x, g, 0.0)
    assert _close(a, OM.moe_ref(wg, wu, wd, xh, res, logits, s, 3)["out"], 0.0)
    assert not np.array_equal(a, OM.moe_ref(wg, wu, wd, xh.astype(F32), res, logits, s, 3)["out"])


def test_moe_norm_tolerance_widens_gate_up_bound():
    OM, wg, wu, wd, x, res, logits, s = _moe_case(seed=42)
    g = np.ones(x.shape[1], F32)
    ref = ON.moe_rmsnorm_ref(wg, wu, wd, x, g, 1e-6, res, logits, s, 2)
    wide = ON.moe_rmsnorm_tolerance(wg, wu, wd, x, g, 1e-6, res, ref)
    narrow = OM.out_tolerance(wg, wu, wd, ON.rmsnorm_ref(x, g, 1e-6), res, ref)
    assert np.all(wide > narrow) and np.all(np.isfinite(wide))
