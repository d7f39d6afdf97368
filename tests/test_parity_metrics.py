"""The error metrics the GPU parity tests use, checked on hand-made arrays."""
import numpy as np

from parity import chunk_rel_err, elementwise_diag, slice_rel_err


def test_chunk_rel_err_normalises_each_chunk():
    ref = np.ones((1, 8, 2, 3))
    ref[:, :4] *= 100.0                  # first chunk (4 steps) 100x larger
    got = ref.copy()
    got[0, 5, 1, 2] += 0.5               # error 0.5 in the small chunk
    # the whole-slice metric sees 0.5 / 100; the per-chunk one 0.5 / 1
    assert np.isclose(slice_rel_err(got, ref, (0, 2)), 5e-3)
    assert np.isclose(chunk_rel_err(got, ref, 4), 0.5)
    # a ragged last chunk (7 steps in chunks of 4) is padded, not dropped
    assert np.isclose(chunk_rel_err(got[:, :7], ref[:, :7], 4), 0.5)
    got[0, 6, 0, 0] = np.nan
    assert chunk_rel_err(got, ref, 4) == float("inf")


def test_elementwise_diag_ignores_entries_below_the_floor():
    ref = np.array([[1000.0, 1.0, 1e-6]])
    got = ref + np.array([[1.0, 0.5, 1.0]])
    # 1e-6 is below 1e-3 * 1000: skipped; 1.0 is at the floor: counted (0.5)
    assert np.isclose(elementwise_diag(got, ref, (0,)), 0.5)
    assert np.isclose(elementwise_diag(got, ref, (0,), floor=0.01), 1e-3)
