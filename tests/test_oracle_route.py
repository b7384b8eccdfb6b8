"""Pins for the oracle's router and permutation: brute force by full sort, a
NumPy stable argsort, and the invariants the tables must satisfy."""
import numpy as np
import pytest

import oracle


def _brute_route(logits, k):
    T, E = logits.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
        ids[t] = order
        sel = np.array([float(logits[t, e]) for e in order])
        ex = np.exp(sel - sel.max())
        w[t] = ex / ex.sum()
    return ids, w


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (33, 64, 8), (17, 256, 8), (9, 5, 5), (4, 40, 32)])
def test_route_brute_force(T, E, k):
    rng = np.random.default_rng(T * 1000 + E)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    # force ties on some rows: values from a tiny set
    logits[: T // 3] = rng.integers(-2, 3, size=(T // 3, E)).astype(np.float32)
    ids, w = oracle.route(logits, k)
    bids, bw = _brute_route(logits, k)
    np.testing.assert_array_equal(ids, bids)
    ulp = np.spacing(np.abs(bw).astype(np.float32)).astype(np.float64)
    assert (np.abs(w.astype(np.float64) - bw) <= ulp).all()


def test_route_invariants():
    rng = np.random.default_rng(5)
    logits = (rng.standard_normal((500, 128)) * 3).astype(np.float32)
    ids, w = oracle.route(logits, 8)
    for t in range(500):
        assert len(set(ids[t].tolist())) == 8
    assert (np.diff(w, axis=1) <= 0).all()
    assert np.abs(w.astype(np.float64).sum(1) - 1.0).max() < 1e-6
    # the picks are the k largest logits
    srt = np.sort(logits, axis=1)[:, ::-1]
    np.testing.assert_array_equal(np.take_along_axis(logits, ids, 1), srt[:, :8])


@pytest.mark.parametrize("k", [1, 2, 4, 8, 16])
def test_route_equal_logits(k):
    logits = np.full((3, 64), 0.7, np.float32)
    ids, w = oracle.route(logits, k)
    np.testing.assert_array_equal(ids, np.tile(np.arange(k, dtype=np.int32), (3, 1)))
    assert (w == np.float32(1.0 / k)).all()


def test_route_rejects_nan():
    lg = np.zeros((2, 8), np.float32)
    lg[1, 3] = np.nan
    with pytest.raises(ValueError):
        oracle.route(lg, 2)


@pytest.mark.parametrize("first_local,E_local", [(0, 64), (64, 64), (192, 64), (0, 256), (7, 1)])
def test_permute_against_stable_argsort(first_local, E_local):
    rng = np.random.default_rng(first_local + E_local)
    T, k, Eg = 300, 8, 256
    logits = rng.standard_normal((T, Eg)).astype(np.float32)
    ids, _ = oracle.route(logits, k)
    counts, offsets, sorted_, inv = oracle.permute(ids, first_local, E_local)
    flat = ids.reshape(-1).astype(np.int64) - first_local
    local = (flat >= 0) & (flat < E_local)
    slots = np.nonzero(local)[0]
    ref_sorted = slots[np.argsort(flat[slots], kind="stable")]
    np.testing.assert_array_equal(sorted_, ref_sorted)
    np.testing.assert_array_equal(counts, np.bincount(flat[local], minlength=E_local))
    assert offsets[0] == 0 and (np.diff(offsets) == counts).all()
    assert offsets[-1] == local.sum() == sorted_.size
    # inv is the inverse map on local slots and -1 elsewhere
    np.testing.assert_array_equal(inv[~local], -1)
    np.testing.assert_array_equal(inv[sorted_], np.arange(sorted_.size))
    # each expert's segment holds only that expert, in increasing slot order
    for e in range(E_local):
        seg = sorted_[offsets[e]:offsets[e + 1]]
        assert (flat[seg] == e).all() and (np.diff(seg) > 0).all()


def test_permute_empty_and_all_nonlocal():
    ids = np.zeros((0, 4), np.int32)
    counts, offsets, sorted_, inv = oracle.permute(ids, 0, 8)
    assert sorted_.size == 0 and (counts == 0).all() and (offsets == 0).all()
    ids = np.full((5, 2), 3, np.int32)
    counts, offsets, sorted_, inv = oracle.permute(ids, 10, 4)
    assert sorted_.size == 0 and (inv == -1).all()
