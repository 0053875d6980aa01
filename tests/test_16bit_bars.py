"""The 16-bit parity bars against 16-bit rounding itself (CPU only).

Against the exact-activation oracle, a 16-bit path can be held to no tighter
bars than rounding its activations allows. The model in tests.rounding_model
applies that rounding to an fp64 copy of the oracle's arithmetic; scaling
the rounded values by factors across a binade (the paths use log2 e in the
filter and 1 in the atom-wise layers) gives different, equally valid samples
of the rounding error. This test checks that the bars in tests.gpu_helpers
admit every sample with room to spare, for the bf16 filter and for W16A16,
on one-, five- and eight-block chain models: a deeper model passes more
rounded values into its forces (the bars are stated for up to five blocks
and scaled by T / 5 beyond), and the one-block model's energies cancel to a
fifth of the sum of its per-atom energies.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from gen.configs import make_config, make_weights
from tests.gpu_helpers import (E_TOL_BF16_ABS_SUM, E_TOL_W16_ABS_SUM, F_RMS_TOL_BF16,
                               F_RMS_TOL_W16, F_TOL_BF16, F_TOL_W16, depth_scale, oracle_desc)
from tests.rounding_model import LOG2E, rounded_energy_forces

MARGIN = 1.25
# (filter scale, atom-wise scale): eight points across a binade, then the paths' own
SCALES = [(2.0 ** (k / 8), 2.0 ** ((3 * k % 8) / 8)) for k in range(8)] + [(LOG2E, 1.0)]
BARS = {1: (E_TOL_BF16_ABS_SUM, F_TOL_BF16, F_RMS_TOL_BF16),
        2: (E_TOL_W16_ABS_SUM, F_TOL_W16, F_RMS_TOL_W16)}


@pytest.mark.parametrize("T", [1, 5, 8])
@pytest.mark.parametrize("dtype", [1, 2])
def test_16bit_bars_admit_rounding(dtype, T):
    """The chain model with one and five blocks; with eight, the largest block
    count, a 63-function basis (the bars then scaled by depth_scale)."""
    cfg, pos, types, _ = make_config("cg269x64", n_replicas=4)
    m = dataclasses.replace(cfg.model, T=T, filter_dtype=dtype)
    if T == 8:
        m = dataclasses.replace(m, Dr=63)
    w = make_weights(m, 11 if T == 8 else 4, bias_scale=0.05)
    desc = oracle_desc(m)
    rp, col = oracle.neighbor_list(pos, 4, 269, False, 0.0, m.r_cut)
    Eo, Fo, eps = oracle.energy_forces(desc, w, pos, types, rp, col, n_replicas=4,
                                       return_eps=True)
    sa = np.abs(eps).reshape(4, -1).sum(axis=1)
    rms = np.sqrt(np.mean(Fo ** 2))
    # without rounding the model is the oracle
    E0, F0, _ = rounded_energy_forces(desc, w, pos, types, rp, col, 4, rnd=False)
    np.testing.assert_allclose(E0, Eo, rtol=1e-11)
    assert np.max(np.abs(F0 - Fo)) <= 1e-10 * rms
    worst = np.zeros(3)
    for c, ca in SCALES:
        E, F, _ = rounded_energy_forces(desc, w, pos, types, rp, col, 4, scale=c, atom_scale=ca)
        err = np.abs(F - Fo)
        got = np.array([np.max(np.abs(E - Eo) / sa), err.max() / rms,
                        np.sqrt(np.mean(err ** 2)) / rms])
        assert got[1] > 1e-4                 # the rounding is in effect
        worst = np.maximum(worst, got)
    print(f"dtype {dtype} T={T}: worst over {len(SCALES)} scales: E err/sum|eps| "
          f"{worst[0]:.2e}, F max/rms {worst[1]:.2e}, F rms/rms {worst[2]:.2e}")
    e_bar, f_bar, f_rms_bar = (depth_scale(T) * b for b in BARS[dtype])
    assert MARGIN * worst[0] <= e_bar
    assert MARGIN * worst[1] <= f_bar
    assert MARGIN * worst[2] <= f_rms_bar
