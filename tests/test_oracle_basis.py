"""Pins for the oracle's elementwise pieces: closed forms and library routines."""
import numpy as np
import pytest
import scipy.special
import torch

from oracle.schnet import (ModelDesc, _bf16_round, cutoff, cutoff_deriv, rbf, rbf_centres,
                           rbf_deriv, sigmoid, ssp)

DESC = ModelDesc(n_types=1, D=8, Dr=50, T=1, rbf_min=0.0, rbf_max=12.0, r_cut=12.0, H=4)


def test_rbf_closed_forms():
    mu, sigma = rbf_centres(DESC)
    assert mu[0] == 0.0 and abs(mu[-1] - 12.0) < 1e-12
    assert abs(sigma - 12.0 / 49) < 1e-15
    for k in (0, 7, 49):
        g = rbf(np.array([mu[k]]), DESC)[0]
        assert abs(g[k] - 1.0) < 1e-15
        gp = rbf(np.array([mu[k] + sigma]), DESC)[0]
        gm = rbf(np.array([mu[k] - sigma]), DESC)[0]
        assert abs(gp[k] - np.exp(-0.5)) < 1e-14
        assert abs(gm[k] - np.exp(-0.5)) < 1e-14
        # neighbouring centre sits one width away
        if k + 1 < 50:
            assert abs(g[k + 1] - np.exp(-0.5)) < 1e-14


def test_cutoff_closed_forms():
    rc = 5.0
    assert cutoff(0.0, rc) == 1.0
    assert abs(cutoff(rc / 2, rc) - 0.5) < 1e-15
    assert cutoff(rc, rc) == 0.0
    assert cutoff(rc + 1.0, rc) == 0.0
    assert abs(cutoff_deriv(rc * (1 - 1e-9), rc)) < 1e-8
    assert abs(cutoff_deriv(rc / 2, rc) + 0.5 * np.pi / rc) < 1e-15


def test_derivatives_against_central_differences():
    d = np.linspace(0.3, 11.7, 41)
    h = 1e-6
    num = (rbf(d + h, DESC) - rbf(d - h, DESC)) / (2 * h)
    assert np.max(np.abs(num - rbf_deriv(d, DESC))) < 1e-7
    numc = (cutoff(d + h, 12.0) - cutoff(d - h, 12.0)) / (2 * h)
    assert np.max(np.abs(numc - cutoff_deriv(d, 12.0))) < 1e-8


def test_ssp_closed_forms_and_library():
    assert ssp(np.array(0.0)) == 0.0
    assert abs(sigmoid(np.array(0.0)) - 0.5) < 1e-16
    assert abs(ssp(np.array(50.0)) - (50.0 - np.log(2.0))) < 1e-12
    assert abs(ssp(np.array(-50.0)) + np.log(2.0)) < 1e-20 + 1e-21
    x = np.linspace(-40, 40, 1001)
    assert np.max(np.abs(ssp(x) - (np.logaddexp(0.0, x) - np.log(2.0)))) < 1e-13
    assert np.max(np.abs(sigmoid(x) - scipy.special.expit(x))) < 1e-15
    h = 1e-6
    num = (ssp(x + h) - ssp(x - h)) / (2 * h)
    assert np.max(np.abs(num - sigmoid(x))) < 1e-8


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    a = (rng.standard_normal(100000) * 10.0 ** rng.uniform(-6, 6, 100000)).astype(np.float32)
    # include exact ties between two bfloat16 neighbours
    ties = (np.arange(1, 1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    a = np.concatenate([a, ties, -ties])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(_bf16_round(a), ref)
