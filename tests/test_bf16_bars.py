"""The bf16-filter parity bars against bf16 rounding itself (CPU only).

Against the exact-activation oracle, the bf16 filter path can be held to no
tighter bars than rounding its filter activations to bf16 allows. The model
in tests.bf16_model applies that rounding to an fp64 copy of the oracle's
arithmetic; scaling the rounded values by factors across a binade (the path
uses log2 e) gives different, equally valid samples of the rounding error.
This test checks that the bars in tests.gpu_helpers admit every sample with
room to spare, for one- and five-block chain models: a deeper model passes
more rounded filter outputs into its forces, and the one-block model's
energies cancel to a fifth of the sum of its per-atom energies.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from gen.configs import make_config, make_weights
from tests.bf16_model import LOG2E, rounded_energy_forces
from tests.gpu_helpers import E_TOL_BF16_ABS_SUM, F_RMS_TOL_BF16, F_TOL_BF16, oracle_desc

MARGIN = 1.25
SCALES = [2.0 ** (k / 8) for k in range(8)] + [LOG2E]


@pytest.mark.parametrize("T", [1, 5])
def test_bf16_bars_admit_rounding(T):
    cfg, pos, types, _ = make_config("cg269x64", n_replicas=4)
    m = dataclasses.replace(cfg.model, T=T, filter_dtype=1)
    w = make_weights(m, 4, bias_scale=0.05)
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
    for c in SCALES:
        E, F, _ = rounded_energy_forces(desc, w, pos, types, rp, col, 4, scale=c)
        err = np.abs(F - Fo)
        got = np.array([np.max(np.abs(E - Eo) / sa), err.max() / rms,
                        np.sqrt(np.mean(err ** 2)) / rms])
        assert got[1] > 1e-3                 # the rounding is in effect
        worst = np.maximum(worst, got)
    print(f"T={T}: worst over {len(SCALES)} scales: E err/sum|eps| {worst[0]:.2e}, "
          f"F max/rms {worst[1]:.2e}, F rms/rms {worst[2]:.2e}")
    assert MARGIN * worst[0] <= E_TOL_BF16_ABS_SUM
    assert MARGIN * worst[1] <= F_TOL_BF16
    assert MARGIN * worst[2] <= F_RMS_TOL_BF16
