"""Pins of the top-K cache-writer oracle against independent routines and invariants (CPU)."""
import heapq

import numpy as np

from chunked_kl_loss_seq_amd import workloads as WL
from oracle import topk_rows


def brute_force(row, K):
    """Pure-Python definition: sort ids by (value descending, id ascending)."""
    ids = sorted(range(len(row)), key=lambda j: (-float(row[j]) + 0.0, j))[:K]
    return ids, [float(row[j]) for j in ids]


def test_matches_pure_python_sort_on_small_rows():
    rng = np.random.default_rng(1)
    for trial in range(40):
        V = int(rng.integers(1, 40))
        K = int(rng.integers(1, V + 1))
        # few distinct values, so ties are frequent
        row = rng.integers(-3, 4, size=V).astype(np.float64) * 0.5
        ids, vals = topk_rows(row[None, :], K)
        bi, bv = brute_force(row, K)
        assert ids[0].tolist() == bi, (row, K)
        assert vals[0].tolist() == bv


def test_matches_heapq():
    rng = np.random.default_rng(2)
    x = WL.round_bf16(rng.standard_normal((6, 3000)).astype(np.float32) * 3)
    ids, vals = topk_rows(x, 100)
    for r in range(6):
        ref = heapq.nsmallest(100, range(3000), key=lambda j: (-float(x[r, j]), j))
        assert ids[r].tolist() == ref


def test_k1_is_argmax_first_occurrence_and_kv_is_full_sort():
    rng = np.random.default_rng(3)
    x = WL.round_bf16(rng.standard_normal((8, 500)).astype(np.float32))
    x[0, 10] = x[0, 20] = x[0].max() + 1  # a tie at the maximum: the lower id wins
    ids, vals = topk_rows(x, 1)
    np.testing.assert_array_equal(ids[:, 0], np.argmax(x, axis=1))
    assert ids[0, 0] == 10
    ids, vals = topk_rows(x, 500)
    for r in range(8):
        assert sorted(ids[r].tolist()) == list(range(500))
        assert np.all(np.diff(vals[r]) <= 0)


def test_all_equal_row_and_signed_zeros_and_infinities():
    ids, vals = topk_rows(np.full((1, 50), 2.5), 7)
    assert ids[0].tolist() == list(range(7)) and np.all(vals == 2.5)
    row = np.array([[0.0, -0.0, -0.0, 0.0, -1.0, np.inf, -np.inf]])
    ids, vals = topk_rows(row, 7)
    # +inf first, then the four zeros in id order (equal values), then -1, then -inf
    assert ids[0].tolist() == [5, 0, 1, 2, 3, 4, 6]
    assert np.signbit(vals[0][2]) and not np.signbit(vals[0][1])  # the values are the inputs' own


def test_selection_invariants_on_bf16_rows_with_ties():
    rng = np.random.default_rng(4)
    V, K = 20000, 100
    x = WL.round_bf16(rng.standard_normal((5, V)).astype(np.float32) * 3)
    ids, vals = topk_rows(x, K)
    for r in range(5):
        sel = ids[r]
        assert len(set(sel.tolist())) == K
        np.testing.assert_array_equal(vals[r], x[r, sel])
        assert np.all(np.diff(vals[r]) <= 0)
        rest = np.setdiff1d(np.arange(V), sel)
        kth = vals[r, -1]
        assert x[r, rest].max() <= kth
        # every id left out with the K-th value is above every selected id with that value
        tied_out = rest[x[r, rest] == kth]
        tied_in = sel[vals[r] == kth]
        if len(tied_out):
            assert tied_in.max() < tied_out.min()
        # equal values inside the selection are in id order
        for v in np.unique(vals[r]):
            run = sel[vals[r] == v]
            assert np.all(np.diff(run) > 0)
