"""The fp32 filter evaluated on fp16 hi/lo pairs (SN_FILTER_F16X2) vs the fp64
oracle of the fp32 model, through the C ABI, at the fp32 bars (energy 1e-5
relative, forces 1e-4 of the force RMS)."""
import dataclasses

import numpy as np
import pytest

from gen.configs import CONFIGS, Config, SystemSpec, make_config, make_weights
from tests.gpu_helpers import gpu_neighbors, lib_desc, lib_system
from tests.test_gpu_energy_forces import check, run_gpu, sparse_clusters

pytestmark = pytest.mark.gpu

F16X2 = 3


def split(cfg):
    return dataclasses.replace(cfg, model=dataclasses.replace(cfg.model, filter_dtype=F16X2))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cg32(gpu_lib, seed):
    """D 64, Dr 32 (one 32-wide basis chunk)."""
    cfg, pos, types, w = make_config("cg32", seed=seed)
    check(gpu_lib, split(cfg), pos, types, w, what=f"f16x2 cg32 seed {seed}")


def test_cg32_with_biases_and_skin_list(gpu_lib):
    cfg, pos, types, w = make_config("cg32", seed=4, bias_scale=0.1)
    check(gpu_lib, split(cfg), pos, types, w, r_list=cfg.model.r_cut + 1.5,
          what="f16x2 cg32 bias+skin")


def test_cg269_four_replicas_biases(gpu_lib):
    """D 128, Dr 50 (two basis chunks, the second ragged)."""
    cfg, pos, types, w = make_config("cg269x64", n_replicas=4, bias_scale=0.05)
    check(gpu_lib, split(cfg), pos, types, w, n_replicas=4, what="f16x2 cg269x4")


def test_cg269x64_full(gpu_lib):
    cfg, pos, types, w = make_config("cg269x64")
    check(gpu_lib, split(cfg), pos, types, w, what="f16x2 cg269x64")


def test_bulk4k_full(gpu_lib):
    """Dr 64, periodic minimum image."""
    cfg, pos, types, w = make_config("bulk4k")
    check(gpu_lib, split(cfg), pos, types, w, what="f16x2 bulk4k")


def test_small_periodic_box_ragged(gpu_lib):
    cfg = CONFIGS["bulk4k"]
    rng = np.random.default_rng(3)
    n, box = 389, 17.9
    pos = rng.uniform(0, box, (n, 3)).astype(np.float32)
    pos[pos >= np.float32(box)] = 0
    types = rng.integers(0, 4, n).astype(np.int32)
    w = make_weights(cfg.model, 5, bias_scale=0.05)
    c2 = Config("box389", SystemSpec("bulk", 1, n, True, box), cfg.model)
    check(gpu_lib, split(c2), pos, types, w, what="f16x2 box389")


def test_compact_chains_long_rows(gpu_lib):
    from gen.systems import rescale_replicas
    cfg, pos, types, w = make_config("cg269x64", n_replicas=4, bias_scale=0.05)
    pos = rescale_replicas(pos, 269, 0.6)
    check(gpu_lib, split(cfg), pos, types, w, n_replicas=4, what="f16x2 cg269x4 compacted x0.6")


def test_md_model_four_replicas(gpu_lib):
    """The MD workload's model (D 128, Dr 50, H 64) with its fp32 weights."""
    cfg, pos, types, w = make_config("md1024", n_replicas=4)
    check(gpu_lib, split(cfg), pos, types, w, n_replicas=4, what="f16x2 md model x4")


@pytest.mark.parametrize("factor", [2.0 ** -18, 1e-3, 3.0])
def test_weight_magnitudes(gpu_lib, factor):
    """Filter weights and biases scaled away from N(0, 1/fan_in): the
    power-of-two scales of weights and activations follow them. (Much larger
    factors make the model itself ill-conditioned: at 30x the fp32 filter
    misses the force bar as well.)"""
    cfg, pos, types, w = make_config("cg269x64", n_replicas=2, bias_scale=0.05)
    m = cfg.model
    w = np.array(w, dtype=np.float32)
    off = m.n_types * m.D
    nf = m.Dr * m.D + m.D + m.D * m.D + m.D    # Wf1, cf1, Wf2, cf2
    per = nf + 2 * (m.D * m.D + m.D)
    for t in range(m.T):
        w[off + t * per: off + t * per + nf] *= np.float32(factor)
    check(gpu_lib, split(cfg), pos, types, w, n_replicas=2, what=f"f16x2 filter x{factor:g}")


def test_sparse_receivers(gpu_lib):
    cfg = CONFIGS["cg32"]
    pos, types = sparse_clusters()
    w = make_weights(cfg.model, 2, bias_scale=0.05)
    c2 = Config("sparse", SystemSpec("chain_walk", 1, len(pos), False), cfg.model)
    check(gpu_lib, split(c2), pos, types, w, what="f16x2 sparse clusters")


def test_isolated_atoms(gpu_lib):
    cfg = CONFIGS["cg32"]
    w = make_weights(cfg.model, 0, bias_scale=0.1)
    pos = (np.arange(12, dtype=np.float32)[:, None] * np.float32(40.0)).repeat(3, 1)
    types = np.zeros(12, np.int32)
    c2 = Config("iso", SystemSpec("chain_walk", 12, 1, False), cfg.model)
    _, F = check(gpu_lib, split(c2), pos, types, w, what="f16x2 12 single-atom replicas")
    assert np.all(F == 0)


def test_two_atom_distance_sweep(gpu_lib):
    """4000 two-atom replicas with the distance swept over (0.3 A, r_c) for
    the narrow-basis bulk model (sigma = 0.079 A) and the chain model: every
    replica's force within the bar of the sweep's force RMS. Rare distances
    put a basis value on a rounding tie; the pair split must still be exact."""
    for name in ("bulk4k", "cg269x64"):
        m = CONFIGS[name].model
        w = make_weights(m, 0)
        R = 4000
        ds = np.linspace(0.3, m.r_cut * 0.995, R)
        rng = np.random.default_rng(1)
        dirs = rng.standard_normal((R, 3))
        dirs /= np.linalg.norm(dirs, axis=1, keepdims=True)
        pos = np.zeros((R, 2, 3))
        pos[:, 0] = rng.uniform(0, 3, (R, 3))
        pos[:, 1] = pos[:, 0] + ds[:, None] * dirs
        pos = pos.reshape(-1, 3).astype(np.float32)
        types = np.tile(np.array([0, 1], np.int32), R)
        c2 = Config("pairs", SystemSpec("chain_walk", R, 2, False), m)
        check(gpu_lib, split(c2), pos, types, w, n_replicas=R, what=f"f16x2 {name} pairs")


def test_deterministic_and_close_to_fp32(gpu_lib):
    """Bitwise reproducible run to run, and within the fp32 bars of the fp32
    MFMA path as well."""
    cfg, pos, types, w = make_config("cg269x64", n_replicas=3)
    m = split(cfg).model
    system = lib_system(gpu_lib, cfg.system, 3)
    E1, F1, _, _ = run_gpu(gpu_lib, m, system, pos, types, w, m.r_cut)
    E2, F2, _, _ = run_gpu(gpu_lib, m, system, pos, types, w, m.r_cut)
    assert np.array_equal(E1, E2) and np.array_equal(F1, F2)
    Ef, Ff, _, _ = run_gpu(gpu_lib, cfg.model, system, pos, types, w, m.r_cut)
    rms = np.sqrt(np.mean(Ff ** 2))
    assert np.max(np.abs(E1 - Ef) / np.abs(Ef)) < 1e-5
    assert np.max(np.abs(F1 - Ff)) < 1e-4 * rms


def test_unfused_pipeline_rejects_it(gpu_lib):
    import torch
    cfg, pos, types, w = make_config("cg32", seed=0)
    m = split(cfg).model
    desc = lib_desc(gpu_lib, m)
    system = lib_system(gpu_lib, cfg.system)
    model = gpu_lib.sn_model_create(desc, w)
    try:
        p, rowptr, col, ne, _ = gpu_neighbors(gpu_lib, system, pos, m.r_cut)
        ws = gpu_lib.Workspace(gpu_lib.sn_unfused_workspace_size(desc, system, ne))
        t = torch.from_numpy(types).cuda()
        energy = torch.empty(1, dtype=torch.float32, device="cuda")
        forces = torch.empty(p.numel(), dtype=torch.float32, device="cuda")
        with pytest.raises(gpu_lib.SnError) as ex:
            gpu_lib.sn_energy_forces_unfused(model, system, p, t, rowptr, col, ne, 0, energy,
                                             forces, ws)
        assert ex.value.status == gpu_lib.SN_ERR_UNSUPPORTED
    finally:
        gpu_lib.sn_model_destroy(model)
