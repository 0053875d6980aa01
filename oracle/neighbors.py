"""Neighbour list oracle: directed edges within a radius, grouped by receiver.

Follows FlashSchNet §3.2 "Building the neighbor list" (directed edges
j = src[e] -> i = dst[e] within the cutoff) and §4.3 "Index construction under
dynamic neighbor lists" (bucket sort by destination into contiguous segments).

Readings taken where the page is silent:
* both directions of every pair, i != j, same replica only;
* strict inequality d < r_list;
* the predicate is evaluated in fp64 on the fp32 inputs without fused
  multiply-add: delta = x_j - x_i per axis; with a periodic cube of side L
  (positions in [0, L)) delta -= L if delta > L/2, delta += L if delta < -L/2;
  s = (dx*dx + dy*dy) + dz*dz; edge iff s < r*r with r the fp64 value of the
  fp32 radius;
* the canonical list is receiver-major with senders ascending inside each
  segment, which is the only list accepted as exact.

Output: ``rowptr`` int64 [R*N + 1] and ``col`` int64 [E]; receiver i owns
``col[rowptr[i]:rowptr[i+1]]``. Atom indices are global (replica-major).
"""
from __future__ import annotations

import numpy as np


def _pair_mask(pi: np.ndarray, pj: np.ndarray, periodic: bool, L: float, r2: float) -> np.ndarray:
    """Predicate for all (i, j) with i from ``pi`` [a,3] and j from ``pj`` [b,3];
    fp64 elementwise numpy arithmetic (no contraction)."""
    s = None
    for ax in range(3):
        d = pj[None, :, ax] - pi[:, None, ax]
        if periodic:
            half = L / 2.0
            d = np.where(d > half, d - L, np.where(d < -half, d + L, d))
        sq = d * d
        s = sq if s is None else s + sq
    return s < r2


def _check(pos, n_replicas, atoms_per_replica, periodic, box, r_list):
    pos = np.asarray(pos)
    if pos.dtype != np.float32 or pos.shape != (n_replicas * atoms_per_replica, 3):
        raise ValueError("pos must be float32 [R*N, 3]")
    L = float(np.float32(box)) if periodic else 0.0
    r = float(np.float32(r_list))
    if periodic:
        if not (L >= 2.0 * r):
            raise ValueError("periodic box must be at least twice the list radius")
        if pos.min() < 0 or pos.max() >= np.float32(box):
            raise ValueError("periodic positions must lie in [0, L)")
    return pos.astype(np.float64), L, r


def neighbor_list_bruteforce(pos, n_replicas, atoms_per_replica, periodic, box, r_list,
                             chunk: int = 2048):
    """O(N^2) per replica. Rows are processed in chunks to bound memory; each
    row's senders come out ascending because columns are scanned in order."""
    p, L, r = _check(pos, n_replicas, atoms_per_replica, periodic, box, r_list)
    N = atoms_per_replica
    r2 = r * r
    counts = np.zeros(n_replicas * N, dtype=np.int64)
    cols = []
    for rep in range(n_replicas):
        base = rep * N
        pr = p[base:base + N]
        for a in range(0, N, chunk):
            m = _pair_mask(pr[a:a + chunk], pr, periodic, L, r2)
            idx = np.arange(a, min(a + chunk, N))
            m[np.arange(len(idx)), idx] = False
            counts[base + a: base + a + len(idx)] = m.sum(axis=1)
            rr, cc = np.nonzero(m)          # row-major order: rows then ascending cols
            cols.append(cc + base)
    rowptr = np.zeros(n_replicas * N + 1, dtype=np.int64)
    np.cumsum(counts, out=rowptr[1:])
    col = np.concatenate(cols) if cols else np.zeros(0, dtype=np.int64)
    return rowptr, col.astype(np.int64)


def neighbor_list_kdtree(pos, n_replicas, atoms_per_replica, periodic, box, r_list):
    """Candidates from scipy's cKDTree within a slightly enlarged radius; the
    exact predicate above decides membership."""
    from scipy.spatial import cKDTree

    p, L, r = _check(pos, n_replicas, atoms_per_replica, periodic, box, r_list)
    N = atoms_per_replica
    r2 = r * r
    rows_all, cols_all = [], []
    for rep in range(n_replicas):
        base = rep * N
        pr = p[base:base + N]
        tree = cKDTree(pr, boxsize=L if periodic else None)
        pairs = tree.query_pairs(r * (1.0 + 1e-6), output_type="ndarray")
        if len(pairs) == 0:
            continue
        i, j = pairs[:, 0], pairs[:, 1]
        s = None
        for ax in range(3):
            d = pr[j, ax] - pr[i, ax]
            if periodic:
                d = np.where(d > L / 2.0, d - L, np.where(d < -L / 2.0, d + L, d))
            sq = d * d
            s = sq if s is None else s + sq
        keep = s < r2
        i, j = i[keep], j[keep]
        rows_all += [i + base, j + base]
        cols_all += [j + base, i + base]
    n_tot = n_replicas * N
    if rows_all:
        rows = np.concatenate(rows_all)
        cols = np.concatenate(cols_all)
        order = np.lexsort((cols, rows))
        rows, cols = rows[order], cols[order]
    else:
        rows = cols = np.zeros(0, dtype=np.int64)
    rowptr = np.zeros(n_tot + 1, dtype=np.int64)
    np.cumsum(np.bincount(rows, minlength=n_tot), out=rowptr[1:])
    return rowptr, cols.astype(np.int64)


def neighbor_list(pos, n_replicas, atoms_per_replica, periodic, box, r_list):
    """Brute force for small replicas, tree candidates for large ones."""
    if atoms_per_replica <= 4096:
        return neighbor_list_bruteforce(pos, n_replicas, atoms_per_replica, periodic, box, r_list)
    return neighbor_list_kdtree(pos, n_replicas, atoms_per_replica, periodic, box, r_list)
