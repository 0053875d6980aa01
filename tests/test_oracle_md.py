"""Pins for the oracle's integrator and noise: numpy's Philox generator, normal
moments, the exact Ornstein-Uhlenbeck limit and velocity Verlet energy
conservation."""
import numpy as np
import pytest

from oracle.md import KAPPA, KB, baoab_run, gaussian_noise, init_velocities, philox4x64_10
from oracle.neighbors import neighbor_list
from oracle.schnet import ModelDesc, energy_forces, unpack_weights
from gen.systems import model_weights


@pytest.mark.parametrize("key", [0, 7, 2**63 + 12345])
def test_philox_matches_numpy_bit_generator(key):
    """numpy's Philox is Philox4x64-10; it increments the 256-bit counter before
    each block, so block b of a generator started at counter c is the function
    evaluated at c + b + 1."""
    start = np.array([5, 2**64 - 1, 3, 0], dtype=np.uint64)
    bg = np.random.Philox(key=np.array([key, 99], dtype=np.uint64), counter=start)
    raw = bg.random_raw(4 * 6).reshape(6, 4)
    ctrs = []
    c = [int(v) for v in start]
    for _ in range(6):
        val = (c[0] + (c[1] << 64) + (c[2] << 128) + (c[3] << 192) + 1) % (1 << 256)
        c = [(val >> (64 * k)) & ((1 << 64) - 1) for k in range(4)]
        ctrs.append(c)
    ours = philox4x64_10(np.array(ctrs, dtype=np.uint64), (key, 99))
    assert np.array_equal(ours, raw)


def test_noise_moments_and_independence():
    z = gaussian_noise(3, 17, np.arange(200000))
    assert z.shape == (200000, 3)
    assert np.all(np.abs(z.mean(axis=0)) < 0.01)
    assert np.all(np.abs(z.var(axis=0) - 1) < 0.015)
    c = np.corrcoef(z.T)
    assert np.max(np.abs(c - np.eye(3))) < 0.01
    # fourth moment of a normal is 3
    assert np.all(np.abs((z ** 4).mean(axis=0) - 3) < 0.06)
    z2 = gaussian_noise(3, 18, np.arange(200000))
    assert abs(np.corrcoef(z[:, 0], z2[:, 0])[0, 1]) < 0.01


def test_zero_force_is_exact_ornstein_uhlenbeck():
    """With zero forces BAOAB's O step is the exact OU update, so velocities
    started from Maxwell-Boltzmann stay at <m v^2 / 2> = 3/2 kB T per atom."""
    n, T, m = 20000, 300.0, 100.0
    v = init_velocities(11, n, T, m)
    pos = np.zeros((n, 3))
    zero = lambda p: (np.zeros(1), np.zeros_like(p))
    _, v2, _, _, _ = baoab_run(zero, lambda p: None, pos, v, np.zeros((n, 3)), dt_fs=2.0,
                                temperature_K=T, gamma_per_ps=50.0, mass_amu=m, skin=1e9,
                                rebuild_every=10**9, seed=11, step0=0, n_steps=50)
    ke = 0.5 * m * np.sum(v2 ** 2, axis=1) / KAPPA            # kcal/mol
    expect = 1.5 * KB * T
    assert abs(ke.mean() / expect - 1) < 0.02
    ke0 = 0.5 * m * np.sum(v ** 2, axis=1) / KAPPA
    assert abs(ke0.mean() / expect - 1) < 0.02


def _chain_system():
    rng = np.random.default_rng(21)
    n = 16
    steps = rng.standard_normal((n - 1, 3))
    steps = 3.8 * steps / np.linalg.norm(steps, axis=1, keepdims=True)
    pos = np.vstack([np.zeros(3), np.cumsum(steps, 0)]).astype(np.float32)
    desc = ModelDesc(n_types=2, D=16, Dr=12, T=2, rbf_min=0.0, rbf_max=8.0, r_cut=8.0, H=8)
    W = unpack_weights(desc, model_weights(np.random.default_rng(3), 2, 16, 12, 2, 8))
    types = rng.integers(0, 2, n).astype(np.int32)
    return desc, W, pos, types


@pytest.mark.slow
def test_velocity_verlet_limit_conserves_energy_to_second_order():
    """gamma = 0 turns BAOAB into velocity Verlet: the total energy error is
    bounded and shrinks about fourfold when dt halves."""
    desc, W, pos, types = _chain_system()
    n = len(pos)
    m = 100.0
    state = {}

    def rebuild(p):
        state["nl"] = neighbor_list(np.asarray(p, np.float32), 1, n, False, 0.0, desc.r_cut + 3.0)

    def forces(p):
        return energy_forces(desc, None, p, types, *state["nl"], weights=W)

    def drift(dt, t_total=400.0):
        rebuild(pos)
        E0, F0 = forces(pos.astype(np.float64))
        v0 = init_velocities(5, n, 300.0, m)
        tot0 = E0[0] + 0.5 * m * np.sum(v0 ** 2) / KAPPA
        p, v, F = pos.astype(np.float64), v0, F0
        errs = []
        for _ in range(int(t_total / dt / 20)):
            p, v, F, E, _ = baoab_run(forces, rebuild, p, v, F, dt_fs=dt, temperature_K=0.0,
                                      gamma_per_ps=0.0, mass_amu=m, skin=3.0, rebuild_every=10,
                                      seed=0, step0=0, n_steps=20)
            errs.append(E[0] + 0.5 * m * np.sum(v ** 2) / KAPPA - tot0)
        return np.max(np.abs(errs))

    e1 = drift(2.0)
    e2 = drift(1.0)
    assert e1 > 0
    assert 2.5 < e1 / e2 < 6.0
