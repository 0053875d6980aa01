"""Pins for the oracle's neighbour list: brute force, tree candidates and an
explicit 27-image search must give the same receiver-sorted list."""
import itertools

import numpy as np
import pytest

from gen.configs import make_config
from oracle.neighbors import neighbor_list_bruteforce, neighbor_list_kdtree


def _images_list(pos, L, r):
    """All ordered pairs (i, j), i != j, whose shortest image distance is
    below r, from an explicit search over the 27 images (valid for L >= 2r)."""
    p = pos.astype(np.float64)
    n = len(p)
    best = np.full((n, n), np.inf)
    for sh in itertools.product((-1, 0, 1), repeat=3):
        dd = p[None, :, :] + np.array(sh) * L - p[:, None, :]
        best = np.minimum(best, np.sqrt(np.sum(dd * dd, axis=-1)))
    np.fill_diagonal(best, np.inf)
    rows, cols = np.nonzero(best < r)
    rowptr = np.zeros(n + 1, dtype=np.int64)
    np.cumsum(np.bincount(rows, minlength=n), out=rowptr[1:])
    return rowptr, cols


def _as_set(rowptr, col):
    dst = np.repeat(np.arange(len(rowptr) - 1), np.diff(rowptr))
    return set(zip(dst.tolist(), np.asarray(col).tolist()))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_periodic_bruteforce_matches_27_images(seed):
    rng = np.random.default_rng(seed)
    L, r, n = 12.0, 3.7, 300
    pos = rng.uniform(0, L, (n, 3)).astype(np.float32)
    rp, col = neighbor_list_bruteforce(pos, 1, n, True, L, r)
    rp2, col2 = _images_list(pos, np.float64(np.float32(L)), np.float64(np.float32(r)))
    # the image search uses a different (sqrt) formula, so compare away from ties
    assert _as_set(rp, col) == _as_set(rp2, col2)


@pytest.mark.parametrize("periodic", [False, True])
@pytest.mark.parametrize("seed", [0, 1])
def test_bruteforce_matches_tree(periodic, seed):
    rng = np.random.default_rng(100 + seed)
    L, r, n = 20.0, 4.0, 2000
    pos = rng.uniform(0, L, (n, 3)).astype(np.float32)
    a = neighbor_list_bruteforce(pos, 2, n // 2, periodic, L, r)
    b = neighbor_list_kdtree(pos, 2, n // 2, periodic, L, r)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_canonical_order_symmetry_and_replicas():
    cfg, pos, types, w = make_config("cg269x64", n_replicas=3)
    rp, col = neighbor_list_bruteforce(pos, 3, 269, False, 0.0, cfg.model.r_cut)
    n = 3 * 269
    dst = np.repeat(np.arange(n), np.diff(rp))
    for i in range(n):
        seg = col[rp[i]:rp[i + 1]]
        assert np.all(np.diff(seg) > 0), "senders ascending inside a segment"
        assert i not in seg
        assert np.all(seg // 269 == i // 269), "edges stay inside a replica"
    assert _as_set(rp, col) == {(j, i) for (i, j) in _as_set(rp, col)}


def test_exact_predicate_at_the_radius():
    """Pairs placed one fp32 ulp inside, at, and outside the radius along an
    axis: the strict inequality keeps only the inside pair."""
    r = np.float32(5.0)
    inside = np.nextafter(r, np.float32(0))
    outside = np.nextafter(r, np.float32(10))
    pos = np.array([[0, 0, 0], [inside, 0, 0],
                    [20, 0, 0], [20 + r, 0, 0],
                    [40, 0, 0], [40 + outside, 0, 0]], dtype=np.float32)
    rp, col = neighbor_list_bruteforce(pos, 1, 6, False, 0.0, r)
    assert _as_set(rp, col) == {(0, 1), (1, 0)}
    rp2, col2 = neighbor_list_kdtree(pos, 1, 6, False, 0.0, r)
    assert np.array_equal(rp, rp2) and np.array_equal(col, col2)


def test_bulk_density_and_tree_at_full_size():
    cfg, pos, types, w = make_config("bulk4k")
    a = neighbor_list_bruteforce(pos, 1, 4096, True, cfg.system.box, cfg.model.r_cut)
    b = neighbor_list_kdtree(pos, 1, 4096, True, cfg.system.box, cfg.model.r_cut)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    mean_deg = len(a[1]) / 4096
    # expected (N-1)/L^3 * 4/3 pi r^3 = 32.04; Poisson spread of the mean is ~0.09
    assert abs(mean_deg - 32.04) < 0.6


def test_periodic_input_checks():
    pos = np.zeros((4, 3), dtype=np.float32)
    with pytest.raises(ValueError):
        neighbor_list_bruteforce(pos, 1, 4, True, 9.0, 5.0)      # box < 2 r
    pos[0, 0] = 10.0
    with pytest.raises(ValueError):
        neighbor_list_bruteforce(pos, 1, 4, True, 10.0, 4.0)     # outside [0, L)
