"""Host-side checks of bench.py: the decode selection read back from the
device is validated before it indexes anything."""
import numpy as np
import pytest

import bench


def test_check_selection_accepts_valid():
    sel = np.array([[[0, 4, 9], [1, 2, 3]]], np.int32)
    assert bench.check_selection(sel, 10, 3).dtype == np.int64


@pytest.mark.parametrize("bad", [[[1, 5, 10]], [[1, 1, 2]], [[-1, 2, 3]], [[3, 2, 1]]])
def test_check_selection_rejects(bad):
    with pytest.raises(RuntimeError):
        bench.check_selection(np.array(bad, np.int32), 10, 3)


def test_check_selection_wrong_count():
    with pytest.raises(RuntimeError):
        bench.check_selection(np.zeros((2, 4), np.int32), 10, 3)
