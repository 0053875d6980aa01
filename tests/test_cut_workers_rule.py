"""Host check of the rule by which the atom-wise kernels and the force sum
find the parts of receivers cut by CFConv worker boundaries (cut_workers in
csrc/tile16.hpp): simulate the partition (worker v starts at edge
16 floor(v T / G), at the receiver holding that edge) and the kernels' tail
rule (a worker holds a part of its last receiver when the next worker's
first receiver started before the next worker's first edge), and compare
the workers holding parts of each receiver with the closed-form range."""
import numpy as np


def _e0(v, T, G, E):
    return min(16 * ((v * T) // G), E)


def _first_receiver(v, T, G, E, rowptr, N):
    if v == G:
        return N
    e = _e0(v, T, G, E)
    lo = int(np.searchsorted(rowptr, e, side="left"))   # first r with rowptr[r] >= e
    return lo - 1 if rowptr[lo] > e else lo


def _holders_simulated(rowptr, N, G):
    E = int(rowptr[N])
    T = (E + 15) // 16
    held = {}
    for w in range(G):
        ia = _first_receiver(w, T, G, E, rowptr, N)
        ia1 = _first_receiver(w + 1, T, G, E, rowptr, N)
        E1 = _e0(w + 1, T, G, E) if w + 1 < G else E
        tail = ia1 < N and rowptr[ia1] < E1
        if ia >= ia1 + (1 if tail else 0):
            continue
        if tail:
            held.setdefault(ia1, []).append(w)
    return held, T


def _holders_closed_form(a, b, T, G):
    if b - a < 2:
        return []
    j0, j1 = a // 16 + 1, (b + 15) // 16
    if j0 >= j1:
        return []
    w0 = (j0 * G + T - 1) // T - 1
    w1 = (j1 * G + T - 1) // T - 1
    return list(range(w0, w1))


def test_cut_worker_ranges_match_the_partition():
    rng = np.random.default_rng(0)
    for trial in range(600):
        N = int(rng.integers(1, 60))
        kind = trial % 3
        if kind == 0:
            deg = rng.integers(0, 40, N)
        elif kind == 1:        # a few long rows among empty ones
            deg = rng.integers(0, 3, N) * rng.integers(0, 200, N)
        else:
            deg = np.where(rng.random(N) < 0.3, 0, rng.integers(1, 20, N))
        rowptr = np.concatenate([[0], np.cumsum(deg)]).astype(np.int64)
        G = int(rng.integers(1, 300))   # also more workers than tiles (empty workers)
        held, T = _holders_simulated(rowptr, N, G)
        for r in range(N):
            got = _holders_closed_form(int(rowptr[r]), int(rowptr[r + 1]), T, G)
            assert got == held.get(r, []), (N, G, r, int(rowptr[r]), int(rowptr[r + 1]))
