"""Langevin molecular dynamics over batched replicas, in fp64.

FlashSchNet §5.1 "Experimental setting" runs Langevin dynamics at 300 K over
parallel replicas and §4.5 "End-to-end integration" lists what one MD step
does (rebuild the neighbour list, rebuild the segment indices, evaluate the
energy, take forces as its negative gradient). The page names no integrator;
the reading taken is BAOAB splitting (Leimkuhler and Matthews, 2013):

  B: v += dt/2 * kappa F / m        A: r += dt/2 * v
  O: v  = c1 v + c2 xi,  c1 = exp(-gamma dt),  c2 = sqrt((1 - c1^2) kB T kappa / m)
  A: r += dt/2 * v      (rebuild list if due)   F = F(r)   B: v += dt/2 * kappa F / m

Units: A, fs, amu, kcal/mol, K. kappa = 4.184e-4 converts kcal/mol/A/amu to
A/fs^2; kB = 0.0019872043 kcal/mol/K.

The noise xi comes from the counter-based generator Philox4x64-10 (Salmon,
Moraes, Dror and Shaw, SC'11), keyed by the seed, one block per atom and step:
counter = (global atom index, step, stream, 0) with stream 0 for the thermostat
and stream 1 for initial velocities; the four 64-bit words become four
uniforms u = ((w >> 11) + 1/2) 2^-53, and Box-Muller turns (u0, u1) and
(u2, u3) into normals, of which the first three are used for x, y, z.
"""
from __future__ import annotations

import numpy as np

KAPPA = 4.184e-4
KB = 0.0019872043

_M0 = np.uint64(0xD2E7470EE14C6C93)
_M1 = np.uint64(0xCA5A826395121157)
_W0 = np.uint64(0x9E3779B97F4A7C15)
_W1 = np.uint64(0xBB67AE8584CAA73B)
_M32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a: np.ndarray, b: np.uint64):
    """Full 64x64 -> 128-bit product of uint64 arrays, as (hi, lo), from 32-bit
    partial products."""
    a_lo, a_hi = a & _M32, a >> _S32
    b_lo, b_hi = b & _M32, b >> _S32
    p_ll = a_lo * b_lo
    p_lh = a_lo * b_hi
    p_hl = a_hi * b_lo
    p_hh = a_hi * b_hi
    mid = (p_ll >> _S32) + (p_lh & _M32) + (p_hl & _M32)
    hi = p_hh + (p_lh >> _S32) + (p_hl >> _S32) + (mid >> _S32)
    lo = a * b
    return hi, lo


def philox4x64_10(counter, key):
    """Philox4x64 with 10 rounds. ``counter`` uint64 [..., 4], ``key`` uint64 [2]
    (broadcast). Returns uint64 [..., 4]."""
    c = np.array(counter, dtype=np.uint64)
    k0 = np.uint64(key[0])
    k1 = np.uint64(key[1])
    x0, x1, x2, x3 = (c[..., i].copy() for i in range(4))
    with np.errstate(over="ignore"):
        for _ in range(10):
            hi0, lo0 = _mulhilo(x0, _M0)
            hi1, lo1 = _mulhilo(x2, _M1)
            x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
            k0 = k0 + _W0
            k1 = k1 + _W1
    return np.stack([x0, x1, x2, x3], axis=-1)


def uniforms(words: np.ndarray) -> np.ndarray:
    """53-bit uniforms in (0, 1): ((w >> 11) + 0.5) * 2^-53."""
    return ((words >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def gaussian_noise(seed: int, step: int, atom_ids, stream: int = 0) -> np.ndarray:
    """Standard normals [len(atom_ids), 3] for one step."""
    atom_ids = np.asarray(atom_ids, dtype=np.uint64)
    ctr = np.zeros((len(atom_ids), 4), dtype=np.uint64)
    ctr[:, 0] = atom_ids
    ctr[:, 1] = np.uint64(step)
    ctr[:, 2] = np.uint64(stream)
    u = uniforms(philox4x64_10(ctr, (np.uint64(seed), np.uint64(0))))
    r01 = np.sqrt(-2.0 * np.log(u[:, 0]))
    r23 = np.sqrt(-2.0 * np.log(u[:, 2]))
    z = np.empty((len(atom_ids), 3))
    z[:, 0] = r01 * np.cos(2.0 * np.pi * u[:, 1])
    z[:, 1] = r01 * np.sin(2.0 * np.pi * u[:, 1])
    z[:, 2] = r23 * np.cos(2.0 * np.pi * u[:, 3])
    return z


def init_velocities(seed: int, n_atoms: int, temperature_K: float, mass_amu: float):
    """Maxwell-Boltzmann velocities in A/fs (stream 1, step 0)."""
    sigma = np.sqrt(KB * temperature_K * KAPPA / mass_amu)
    return sigma * gaussian_noise(seed, 0, np.arange(n_atoms), stream=1)


def baoab_run(forces_fn, rebuild_fn, pos, vel, forces, *, dt_fs, temperature_K, gamma_per_ps,
              mass_amu, skin, rebuild_every, seed, step0, n_steps, periodic=False, box=0.0):
    """Advance ``n_steps`` BAOAB steps.

    ``forces_fn(pos) -> (E[R], F[N,3])`` evaluates the model on the current
    neighbour list; ``rebuild_fn(pos)`` rebuilds that list. The list is rebuilt
    after the drift of step k when (k + 1) is a multiple of ``rebuild_every``
    or when some atom moved more than skin/2 since the last rebuild.
    Returns (pos, vel, forces, energies, n_rebuilds)."""
    pos = np.array(pos, dtype=np.float64)
    vel = np.array(vel, dtype=np.float64)
    F = np.array(forces, dtype=np.float64)
    n = len(pos)
    atom_ids = np.arange(n)
    c1 = np.exp(-gamma_per_ps * 1e-3 * dt_fs)
    c2 = np.sqrt((1.0 - c1 * c1) * KB * temperature_K * KAPPA / mass_amu)
    half_kick = 0.5 * dt_fs * KAPPA / mass_amu
    pos_build = pos.copy()
    E = None
    n_rebuilds = 0
    L = float(np.float32(box)) if periodic else 0.0
    for s in range(n_steps):
        k = step0 + s
        vel += half_kick * F
        pos += 0.5 * dt_fs * vel
        vel = c1 * vel + c2 * gaussian_noise(seed, k, atom_ids, stream=0)
        pos += 0.5 * dt_fs * vel
        if periodic:
            pos -= L * np.floor(pos / L)
        disp = pos - pos_build
        if periodic:
            disp -= L * np.round(disp / L)
        moved = np.sqrt(np.max(np.einsum("ij,ij->i", disp, disp))) if n else 0.0
        if (k + 1) % rebuild_every == 0 or moved > 0.5 * skin:
            rebuild_fn(pos)
            pos_build = pos.copy()
            n_rebuilds += 1
        E, F = forces_fn(pos)
        vel += half_kick * F
    return pos, vel, F, E, n_rebuilds
