"""Seeded synthetic systems and weights.

Workload shapes follow the FlashSchNet page (§5.1 "Experimental setting": 64
replicas of a 269-bead coarse-grained protein) and the TensorNet page (§1
"Where the time goes", Figure 2: 4096 atoms, 5 A cutoff, about 32 neighbours).
The real proteins and trained weights are not available, so seeded stand-ins
with the same sizes and densities are drawn here.

Streams: ``np.random.default_rng([seed, k])`` with k = 0 geometry, 1 types,
2 weights, so that changing one draw never shifts another.
"""
from __future__ import annotations

import numpy as np


def _unit_vectors(rng: np.random.Generator, n: int) -> np.ndarray:
    v = rng.standard_normal((n, 3))
    return v / np.linalg.norm(v, axis=1, keepdims=True)


def chain_walk(rng: np.random.Generator, n_beads: int, step: float = 3.8,
               jitter: float = 0.2) -> np.ndarray:
    """Random walk from the origin with fixed step length, then iid normal
    jitter of the given width on every coordinate. Returns float32 [n, 3]."""
    steps = _unit_vectors(rng, n_beads - 1) * step
    pos = np.zeros((n_beads, 3))
    pos[1:] = np.cumsum(steps, axis=0)
    pos += rng.normal(0.0, jitter, size=pos.shape)
    return pos.astype(np.float32)


def self_avoiding_chain(rng: np.random.Generator, n_beads: int, step: float = 3.8,
                        min_dist: float = 4.0, max_tries: int = 1000) -> np.ndarray:
    """Random walk with fixed step length that rejects a proposal closer than
    ``min_dist`` to any earlier bead except its bonded predecessor. After
    ``max_tries`` rejections in a row the chain restarts (same stream).
    Returns float32 [n, 3]."""
    md2 = min_dist * min_dist
    while True:
        pos = np.zeros((n_beads, 3))
        ok = True
        for k in range(1, n_beads):
            for _ in range(max_tries):
                cand = pos[k - 1] + _unit_vectors(rng, 1)[0] * step
                if k < 2:
                    break
                dd = pos[: k - 1] - cand
                if np.min(np.einsum("ij,ij->i", dd, dd)) >= md2:
                    break
            else:
                ok = False
                break
            pos[k] = cand
        if ok:
            return pos.astype(np.float32)


def rescale_replicas(pos: np.ndarray, n_per: int, factor: float) -> np.ndarray:
    """Each replica's positions scaled by ``factor`` about its own centroid
    (below 1 a more compact conformation with more, and longer-range,
    contacts; above 1 a more extended one). Returns float32 [R*N, 3]."""
    p = np.asarray(pos, dtype=np.float64).reshape(-1, n_per, 3)
    c = p.mean(axis=1, keepdims=True)
    return np.ascontiguousarray((c + factor * (p - c)).reshape(-1, 3), dtype=np.float32)


def bulk_uniform(rng: np.random.Generator, n_atoms: int, box: float) -> np.ndarray:
    """Uniform positions in the periodic cube [0, box)^3, float32. A coordinate
    that rounds up to ``box`` in float32 is set to 0 so that every value lies
    in [0, box)."""
    p = rng.uniform(0.0, box, size=(n_atoms, 3)).astype(np.float32)
    p[p >= np.float32(box)] = 0.0
    return p


def n_model_weights(n_types: int, D: int, Dr: int, T: int, H: int) -> int:
    """Length of the flat weight vector (layout in ``model_weights``)."""
    per_block = Dr * D + D + D * D + D + D * D + D + D * D + D
    return n_types * D + T * per_block + D * H + H + H + 1


def model_weights(rng: np.random.Generator, n_types: int, D: int, Dr: int, T: int,
                  H: int, bias_scale: float = 0.0) -> np.ndarray:
    """Flat float32 weight vector, fan_in-scaled normals.

    Order: Emb[n_types][D]; for each block t: Wf1[Dr][D], cf1[D], Wf2[D][D],
    cf2[D], Wu1[D][D], cu1[D], Wu2[D][D], cu2[D]; then Wo1[D][H], co1[H],
    Wo2[H], co2[1]. Matrices are row-major [fan_in][fan_out].

    The embedding rows are N(0, 1) (a one-hot lookup has fan_in 1). Every
    weight matrix is N(0, 1/fan_in). Biases are zero unless ``bias_scale`` is
    given, in which case they are N(0, bias_scale^2).
    """
    def mat(fi, fo):
        return rng.normal(0.0, 1.0 / np.sqrt(fi), size=(fi, fo))

    def bias(n):
        if bias_scale == 0.0:
            return np.zeros(n)
        return rng.normal(0.0, bias_scale, size=n)

    parts = [rng.normal(0.0, 1.0, size=(n_types, D))]
    for _ in range(T):
        parts += [mat(Dr, D), bias(D), mat(D, D), bias(D),
                  mat(D, D), bias(D), mat(D, D), bias(D)]
    parts += [mat(D, H), bias(H), mat(H, 1), bias(1)]
    flat = np.concatenate([p.ravel() for p in parts]).astype(np.float32)
    assert flat.size == n_model_weights(n_types, D, Dr, T, H)
    return flat


def cell_order(pos, box, cell=5.0):
    """A relabelling of the atoms of one periodic cube: their order by cell of
    the grid of cells of side >= `cell` (z-major, then y, then x; stable
    inside a cell), as an index array."""
    nc = max(1, int(box // cell))
    c = np.floor(pos.astype(np.float64) / (box / nc)).astype(np.int64).clip(0, nc - 1)
    return np.argsort((c[:, 2] * nc + c[:, 1]) * nc + c[:, 0], kind="stable")
