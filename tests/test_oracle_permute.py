"""Pins for the oracle's permutation (CPU only): brute force by a Python sort of
(expert, token, slot) triples, and the invariants of a stable grouping."""
import numpy as np
import pytest

from moe_inputs.generate import routing_with_counts
from oracle.permute import permute


def brute(idx, E):
    T, k = idx.shape
    trip = sorted((int(idx[t, j]), t, j) for t in range(T) for j in range(k))
    src = [t * k + j for (_, t, j) in trip]
    split = [sum(1 for (e, _, _) in trip if e == ee) for ee in range(E)]
    rmap = [0] * (T * k)
    for r, s in enumerate(src):
        rmap[s] = r
    return np.array(split), np.array(src), np.array(rmap)


@pytest.mark.parametrize("T,k,E,seed", [(1, 1, 1, 0), (7, 2, 3, 1), (50, 2, 8, 2), (64, 4, 16, 3), (33, 8, 64, 4)])
def test_brute_force(T, k, E, seed):
    g = np.random.default_rng(seed)
    idx = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    p = permute(idx, E)
    split, src, rmap = brute(idx, E)
    np.testing.assert_array_equal(p.split_sizes, split)
    np.testing.assert_array_equal(p.src_index, src)
    np.testing.assert_array_equal(p.row_id_map, rmap)
    assert p.offsets[0] == 0 and p.offsets[-1] == T * k
    np.testing.assert_array_equal(np.diff(p.offsets), split)


def test_invariants_with_empty_experts():
    counts = [0, 3, 0, 31, 33, 1, 0, 60]       # zero-token experts first, middle, last
    T, k = 64, 2
    idx, _ = routing_with_counts(counts, T, k, seed=5)
    p = permute(idx, len(counts))
    np.testing.assert_array_equal(p.split_sizes, counts)
    assert p.split_sizes.sum() == T * k
    # bijection onto [0, R)
    assert sorted(p.row_id_map.tolist()) == list(range(T * k))
    np.testing.assert_array_equal(p.src_index[p.row_id_map], np.arange(T * k))
    # each row lies in its expert's group, and groups are in ascending (t, j)
    flat = idx.reshape(-1)
    for e in range(len(counts)):
        rows = np.arange(p.offsets[e], p.offsets[e + 1])
        assert np.all(flat[p.src_index[rows]] == e)
        assert np.all(np.diff(p.src_index[rows]) > 0)


def test_out_of_range_rejected():
    with pytest.raises(ValueError):
        permute(np.array([[0, 4]], dtype=np.int32), 4)
