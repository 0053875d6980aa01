"""The cutout used to sample the oracle's forces on boxes too large for a
full evaluation (tests.gpu_helpers.cutout_forces) reproduces the full
periodic oracle exactly inside its guaranteed radius, and visibly fails
beyond it (so the radius rule is what makes it exact)."""
import dataclasses

import numpy as np

import oracle
from gen.configs import make_config, make_weights
from tests.gpu_helpers import cutout_forces, oracle_desc


def test_cutout_is_exact_inside_its_radius():
    cfg, pos, types, _ = make_config("bulk4k")
    m = dataclasses.replace(cfg.model, T=1)          # forces reach 2 T r_c = 10 A
    cfg = dataclasses.replace(cfg, model=m)
    w = make_weights(m, 0, bias_scale=0.05)
    rp, col = oracle.neighbor_list(pos, 1, len(pos), True, cfg.system.box, m.r_cut)
    _, F = oracle.energy_forces(oracle_desc(m), w, pos, types, rp, col, periodic=True,
                                box=cfg.system.box)
    rms = np.sqrt(np.mean(F ** 2))
    atoms, Fc = cutout_forces(cfg, pos, types, w, m, 7, 20.0, 9.9)
    assert len(atoms) > 100
    assert np.max(np.abs(F[atoms] - Fc)) <= 1e-12 * rms
    atoms, Fc = cutout_forces(cfg, pos, types, w, m, 7, 20.0, 19.0)
    assert np.max(np.abs(F[atoms] - Fc)) > 1e-3 * rms
