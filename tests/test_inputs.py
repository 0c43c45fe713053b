"""Host logic of the seeded input generators (no GPU): layouts and list invariants.

The extra-positive lists they draw must pass the same checks the library applies
(increasing columns in [0, N), never the row's own positive), so the oracle's list
validator is used as the reference here."""

import numpy as np
import pytest

from contrastive_embedding_loss_amd.inputs import (
    WORKLOADS, band_lists, bf16_bits_to_f32, make_band_inputs, random_positive_lists, workload_positives)
from oracle.contrastive import check_positives


@pytest.mark.parametrize("R,m,h", [(1, 0, 0), (7, 1, 2), (40, 2, 2), (33, 3, 0)])
def test_band_layout(R, m, h):
    row_ptr, col, N = band_lists(R, m, h)
    counts = np.diff(row_ptr)
    assert np.array_equal(counts, np.arange(R) % (2 * m + 1))
    assert N == R + counts.sum() + R * h
    check_positives((row_ptr, col), R, N, 0, False)
    # entry i's appended keys: its positives first, then its hard negatives, in entry order
    first = R
    for i in range(R):
        assert list(col[row_ptr[i]:row_ptr[i + 1]]) == list(range(first, first + counts[i]))
        first += counts[i] + h
    assert first == N


def test_band_inputs_shapes_and_pairs():
    qb, kb, row_ptr, col = make_band_inputs(12, 64, 2, 1, noise=0.1, hard_noise=2.0, seed=3)
    rp2, col2, N = band_lists(12, 2, 1)
    assert qb.shape == (12, 64) and kb.shape == (N, 64)
    assert np.array_equal(row_ptr, rp2) and np.array_equal(col, col2)
    q, k = bf16_bits_to_f32(qb).astype(np.float64), bf16_bits_to_f32(kb).astype(np.float64)
    # listed positives sit near their entry's query (small noise); hard negatives farther
    for i in range(12):
        for j in col[row_ptr[i]:row_ptr[i + 1]]:
            assert np.linalg.norm(k[j] - q[i]) < 0.25 * np.linalg.norm(q[i])


@pytest.mark.parametrize("R,N,off,mean,dense", [(30, 90, 40, 5.0, None), (30, 90, 0, 5.0, 4), (64, 64, 0, 60.0, 0)])
def test_random_lists_two_set(R, N, off, mean, dense):
    row_ptr, col = random_positive_lists(R, N, off, mean, seed=9, dense_row=dense)
    check_positives((row_ptr, col), R, N, off, False)
    if dense is not None:
        assert row_ptr[dense + 1] - row_ptr[dense] == N - 1


@pytest.mark.parametrize("N,R,off", [(40, 40, 0), (40, 16, 8)])
def test_random_lists_oneset_are_symmetric(N, R, off):
    full_rp, full_col = random_positive_lists(N, N, 0, 4.0, seed=11, oneset=True)
    check_positives((full_rp, full_col), N, N, 0, True)
    pairs = {(i, int(j)) for i in range(N) for j in full_col[full_rp[i]:full_rp[i + 1]]}
    assert pairs == {(j, i) for i, j in pairs}
    rp, col = random_positive_lists(R, N, off, 4.0, seed=11, oneset=True)
    check_positives((rp, col), R, N, off, True)
    for i in range(R):  # a share holds its rows' lists of the same set-wide draw
        assert list(col[rp[i]:rp[i + 1]]) == list(full_col[full_rp[off + i]:full_rp[off + i + 1]])


def test_workload_positives():
    w = WORKLOADS["siglip_band_16384"]
    row_ptr, col = workload_positives(w)
    assert row_ptr.shape == (w.R + 1,) and int(row_ptr[-1]) == len(col) == 32766
    assert int(col.max()) < w.N
    assert workload_positives(WORKLOADS["infonce_32768"]) is None
