"""Host-side logic of bench.py (no GPU): the benchmark hands x to the
library with its own batch argument, so every workload must produce x with
exactly that many rows of its matrix's columns (a shorter x would be read
past its end)."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("workload,batches", [("small", (1, 17, 256)), ("square", (1, 64)), ("layer", (256,))])
def test_workload_x_has_the_requested_batch(workload, batches):
    for batch in batches:
        mats, x = bench.load_workload(workload, batch)
        assert x.shape == (batch, mats[0].shape[1]), (workload, batch, x.shape)


def test_banded_x_extends_the_workload_draw():
    """The banded workload's own x has 16 rows; a larger batch extends the
    same draw."""
    import numpy as np
    import synth
    d = synth.banded()
    mats, x = bench.load_workload("banded", 64)
    assert x.shape == (64, mats[0].shape[1])
    assert np.array_equal(x[:16], d["X"])
