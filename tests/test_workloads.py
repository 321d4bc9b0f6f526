"""The seeded generators: shapes, reproducibility and the distributions the
recipes state (no method arithmetic lives there)."""
import numpy as np
import pytest
from scipy import stats

import workloads


def test_numpy_student_t_moments_and_tail():
    w = workloads.student_t_weights(512, 1024, 0, 1).astype(np.float64) / 0.02
    assert abs(w.var() - 5.0 / 3.0) < 0.05
    assert abs(np.mean(np.abs(w) > 4.0) - 2 * stats.t(5).sf(4.0)) < 0.002
    np.testing.assert_array_equal(workloads.student_t_weights(3, 5, 7, 9), workloads.student_t_weights(3, 5, 7, 9))


def test_device_student_t_distribution_on_cpu():
    torch = pytest.importorskip("torch")
    w = workloads.student_t_weights_device(1000, 1000, 0, 1, device="cpu").numpy().astype(np.float64) / 0.02
    assert w.dtype == np.float64 and w.shape == (1000, 1000)
    assert abs(w.mean()) < 0.01
    assert abs(w.var() - 5.0 / 3.0) < 0.05
    assert abs(np.mean(np.abs(w) > 4.0) - 2 * stats.t(5).sf(4.0)) < 0.001
    # Kolmogorov-Smirnov against Student-t(5) on a subsample
    assert stats.kstest(w.ravel()[:20000], stats.t(5).cdf).pvalue > 1e-3
    a = workloads.student_t_weights_device(4, 4, 3, 5, device="cpu")
    b = workloads.student_t_weights_device(4, 4, 3, 5, device="cpu")
    assert torch.equal(a, b)
    assert not torch.equal(a, workloads.student_t_weights_device(4, 4, 3, 6, device="cpu"))


def test_device_normal_on_cpu():
    pytest.importorskip("torch")
    x = workloads.normal_device((200, 500), 0, 2, device="cpu").numpy().astype(np.float64)
    assert abs(x.mean()) < 0.02 and abs(x.var() - 1.0) < 0.03
