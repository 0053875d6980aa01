"""Pins of the oracle's 16-bit weight path (FlashSchNet §4.4 "W16A16 mixed
precision for MLP submodules", "Channel-wise quantization"): per-output-channel
power-of-two scales and IEEE half-precision rounding, checked against values
worked out by hand from the binary16 format (10 fraction bits, round to
nearest even) and against the format's error bound."""
import dataclasses

import numpy as np

from oracle.neighbors import neighbor_list
from oracle.schnet import W16A16, ModelDesc, energy, energy_forces, f16_channel_quantize, unpack_weights
from gen.systems import model_weights


def test_hand_worked_columns():
    # column 0: largest magnitude 0.7 = 0.7 * 2^0 -> scale 1;
    #   0.3 = 1.2 * 2^-2: fraction 0.2 * 1024 = 204.8 -> 205 -> 0.300048828125
    #   0.7 = 1.4 * 2^-1: 0.4 * 1024 = 409.6 -> 410 -> 0.7001953125
    #   0.1 = 1.6 * 2^-4: 0.6 * 1024 = 614.4 -> 614 -> 0.0999755859375
    # column 1: largest 5 = 0.625 * 2^3 -> scale 8; 3/8 and 5/8 are exact; 0 stays 0
    # column 2: all zero -> scale 1 -> zeros
    # column 3: largest 2e-3 = 0.512 * 2^-8 -> scale 2^-8; 1e-3 / 2^-8 = 0.256
    #   = 1.024 * 2^-2: 0.024 * 1024 = 24.576 -> 25 -> 0.256103515625 (times 2^-8);
    #   2e-3 / 2^-8 = 0.512 = 1.024 * 2^-1 -> 25 -> 0.51220703125 (times 2^-8);
    #   -5e-4 / 2^-8 = -0.128 = -1.024 * 2^-3 -> -0.1280517578125 (times 2^-8)
    W = np.array([[0.3, 3.0, 0.0, 1e-3],
                  [-0.7, 5.0, 0.0, 2e-3],
                  [0.1, 0.0, 0.0, -5e-4]], dtype=np.float32)
    q = f16_channel_quantize(W)
    s3 = 2.0 ** -8
    want = np.array([[0.300048828125, 3.0, 0.0, 0.256103515625 * s3],
                     [-0.7001953125, 5.0, 0.0, 0.51220703125 * s3],
                     [0.0999755859375, 0.0, 0.0, -0.1280517578125 * s3]])
    assert np.array_equal(q.astype(np.float64), want.astype(np.float32).astype(np.float64))


def test_vector_is_one_column():
    v = np.array([0.3, -0.7, 0.1], dtype=np.float32)
    assert np.array_equal(f16_channel_quantize(v), f16_channel_quantize(v[:, None])[:, 0])


def test_grid_scale_and_error_bound():
    rng = np.random.default_rng(5)
    W = (rng.standard_normal((96, 40)) * np.exp(rng.uniform(-12, 6, 40))).astype(np.float32)
    q = f16_channel_quantize(W)
    for n in range(W.shape[1]):
        amax = np.max(np.abs(W[:, n]))
        s = 2.0 ** np.ceil(np.log2(amax))
        if s == amax:              # an exact power of two goes one binade up
            s *= 2.0
        r = q[:, n].astype(np.float64) / s
        # every stored value is a binary16 number below 1 in magnitude ...
        assert np.array_equal(r.astype(np.float16).astype(np.float64), r)
        assert np.max(np.abs(r)) < 1.0 and np.max(np.abs(r)) >= 0.5 - 2.0 ** -12
        # ... within half a unit of the last place of [0.5, 1) (2^-12) of W / s
        assert np.max(np.abs(q[:, n] - W[:, n]) / s) <= 2.0 ** -12


def test_representable_weights_are_unchanged():
    rng = np.random.default_rng(6)
    r = rng.uniform(-1, 1, (64, 16)).astype(np.float16).astype(np.float32)
    r[0] = 0.75                    # every column's largest magnitude in [0.5, 1)
    scales = np.ldexp(np.float32(1.0), rng.integers(-10, 10, 16)).astype(np.float32)
    W = r * scales
    assert np.array_equal(f16_channel_quantize(W), W)


def _small(filter_dtype):
    rng = np.random.default_rng(3)
    n = 20
    steps = rng.standard_normal((n - 1, 3))
    steps = 3.8 * steps / np.linalg.norm(steps, axis=1, keepdims=True)
    pos = np.vstack([np.zeros(3), np.cumsum(steps, 0)]).astype(np.float32)
    desc = ModelDesc(n_types=3, D=32, Dr=12, T=2, rbf_min=0.0, rbf_max=10.0, r_cut=10.0, H=32,
                     filter_dtype=filter_dtype)
    w = model_weights(np.random.default_rng([3, 2]), 3, 32, 12, 2, 32, bias_scale=0.05)
    types = rng.integers(0, 3, n).astype(np.int32)
    return desc, w, pos, types


def test_every_mlp_weight_and_nothing_else_is_quantized():
    desc, w, _, _ = _small(W16A16)
    Wq = unpack_weights(desc, w)
    Wf = unpack_weights(dataclasses.replace(desc, filter_dtype=0), w)
    for t in range(desc.T):
        for name in ("Wf1", "Wf2", "Wu1", "Wu2"):
            assert np.array_equal(Wq["blocks"][t][name],
                                  f16_channel_quantize(Wf["blocks"][t][name]))
            assert not np.array_equal(Wq["blocks"][t][name], Wf["blocks"][t][name])
        for name in ("cf1", "cf2", "cu1", "cu2"):
            assert np.array_equal(Wq["blocks"][t][name], Wf["blocks"][t][name])
    for name in ("Wo1", "Wo2"):
        assert np.array_equal(Wq[name], f16_channel_quantize(Wf[name]))
    for name in ("emb", "co1", "co2"):
        assert np.array_equal(Wq[name], Wf[name])


def test_quantized_model_forces_match_central_differences():
    desc, w, pos, types = _small(W16A16)
    rp, col = neighbor_list(pos, 1, len(pos), False, 0.0, desc.r_cut + 1.0)
    W = unpack_weights(desc, w)
    _, F = energy_forces(desc, None, pos, types, rp, col, weights=W)
    p64 = pos.astype(np.float64)
    h = 1e-5
    num = np.zeros_like(p64)
    for i in range(len(p64)):
        for ax in range(3):
            pp, pm = p64.copy(), p64.copy()
            pp[i, ax] += h
            pm[i, ax] -= h
            num[i, ax] = -(energy(desc, None, pp, types, rp, col, weights=W)[0]
                           - energy(desc, None, pm, types, rp, col, weights=W)[0]) / (2 * h)
    assert np.max(np.abs(num - F)) < 1e-7 * max(np.sqrt(np.mean(F ** 2)), 1.0)
    # 16-bit weights move the energy by about their rounding (2^-12 relative)
    Ef = energy(dataclasses.replace(desc, filter_dtype=0), w, pos, types, rp, col)
    Eq = energy(desc, w, pos, types, rp, col)
    assert 0 < abs(Eq[0] - Ef[0]) < 1e-2 * abs(Ef[0])
