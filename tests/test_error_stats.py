"""The parity tests' error measures, checked on the CPU against values worked
out by hand: the per-tensor bar max|g - o| / max|o| and the element-wise
statistics against max(|o|, 1e-3 max|o|)."""
import numpy as np
import pytest

from tests.gpu_util import ELEM_FLOOR, elem_stats, max_rel


def test_per_tensor_bar():
    assert max_rel([1.0, 2.0, 3.0], [1.0, 2.0, 4.0]) == pytest.approx(0.25)
    assert max_rel([0.0], [0.0]) == 0.0


def test_elementwise_floor_and_percentiles():
    ref = np.array([1.0, 2.1, 0.001, 0.0])
    got = np.array([1.0, 2.0, 0.0, 1e-9])
    floor = ELEM_FLOOR * 2.1
    want = np.array([0.0, 0.1 / 2.1, 0.001 / floor, 1e-9 / floor])
    s = elem_stats(got, ref)
    assert s["max"] == pytest.approx(want.max())
    assert s["median"] == pytest.approx(np.median(want))
    assert s["p99"] == pytest.approx(np.percentile(want, 99))
