"""The unfused pipeline (sn_energy_forces_unfused) vs the fp64 oracle, in both
aggregation modes, through the C ABI."""
import numpy as np
import pytest

import oracle
from gen.configs import CONFIGS, Config, SystemSpec, make_config, make_weights
from tests.gpu_helpers import (assert_energy_forces, gpu_neighbors, lib_desc, lib_system,
                               oracle_desc, oracle_list)

pytestmark = pytest.mark.gpu

MODES = {"segmented": 0, "atomic": 1}


def run_unfused(lib, m, system, pos, types, w, r_list, flags, cap_slack=64, cap=None):
    import torch
    desc = lib_desc(lib, m)
    model = lib.sn_model_create(desc, w)
    try:
        p, rowptr, col, ne, _ = gpu_neighbors(lib, system, pos, r_list)
        cap = ne + cap_slack if cap is None else cap
        ws = lib.Workspace(lib.sn_unfused_workspace_size(desc, system, cap))
        t = torch.from_numpy(np.ascontiguousarray(types, dtype=np.int32)).cuda()
        energy = torch.empty(system.n_replicas, dtype=torch.float32, device="cuda")
        forces = torch.empty(p.numel(), dtype=torch.float32, device="cuda")
        lib.sn_energy_forces_unfused(model, system, p, t, rowptr, col, cap, flags, energy, forces,
                                     ws)
        torch.cuda.synchronize()
        status = lib.sn_get_device_status(ws)
        return (energy.cpu().double().numpy(), forces.cpu().double().numpy().reshape(-1, 3),
                rowptr.cpu().numpy(), col[:ne].cpu().numpy(), status)
    finally:
        lib.sn_model_destroy(model)


def check(lib, cfg, pos, types, w, mode, r_list=None, n_replicas=None, what=""):
    m = cfg.model
    system = lib_system(lib, cfg.system, n_replicas)
    r_list = m.r_cut if r_list is None else r_list
    E, F, rp_gpu, col_gpu, status = run_unfused(lib, m, system, pos, types, w, r_list, MODES[mode])
    assert status[0] == 0, f"device status {status}"
    rp, col = oracle_list(system, pos, r_list, rp_gpu, col_gpu, what)
    Eo, Fo, eps = oracle.energy_forces(oracle_desc(m), w, pos, types, rp, col,
                                       n_replicas=system.n_replicas,
                                       periodic=bool(system.periodic), box=system.box,
                                       return_eps=True)
    re, rf = assert_energy_forces(E, F, Eo, Fo, bf16=m.filter_dtype in (1, 2), what=f"{what} {mode}",
                                  eps_abs_sum=np.abs(eps).reshape(system.n_replicas, -1).sum(axis=1))
    print(f"{what} {mode}: E rel {re:.2e}, F max/rms {rf:.2e}, edges {len(col)}")
    return E, F


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("seed", [0, 1])
def test_cg32(gpu_lib, seed, mode):
    cfg, pos, types, w = make_config("cg32", seed=seed)
    check(gpu_lib, cfg, pos, types, w, mode, what=f"cg32 seed {seed}")


@pytest.mark.parametrize("mode", list(MODES))
def test_cg32_with_biases_and_skin_list(gpu_lib, mode):
    """Nonzero biases and listed edges beyond the cutoff: the mask must remove
    the bias-driven filter of those edges in both passes."""
    cfg, pos, types, w = make_config("cg32", seed=4, bias_scale=0.1)
    check(gpu_lib, cfg, pos, types, w, mode, r_list=cfg.model.r_cut + 1.5, what="cg32 bias+skin")


@pytest.mark.parametrize("mode", list(MODES))
def test_cg269_four_replicas(gpu_lib, mode):
    cfg, pos, types, w = make_config("cg269x64", n_replicas=4, bias_scale=0.05)
    check(gpu_lib, cfg, pos, types, w, mode, n_replicas=4, what="cg269x4")


@pytest.mark.parametrize("mode", list(MODES))
def test_compact_chains_long_rows(gpu_lib, mode):
    from gen.systems import rescale_replicas
    cfg, pos, types, w = make_config("cg269x64", n_replicas=4, bias_scale=0.05)
    pos = rescale_replicas(pos, 269, 0.4)
    check(gpu_lib, cfg, pos, types, w, mode, n_replicas=4, what="cg269x4 compacted x0.4")


@pytest.mark.parametrize("mode", list(MODES))
def test_small_periodic_box_ragged(gpu_lib, mode):
    cfg = CONFIGS["bulk4k"]
    rng = np.random.default_rng(3)
    n, box = 389, 17.9
    pos = rng.uniform(0, box, (n, 3)).astype(np.float32)
    pos[pos >= np.float32(box)] = 0
    types = rng.integers(0, 4, n).astype(np.int32)
    w = make_weights(cfg.model, 5, bias_scale=0.05)
    c2 = Config("box389", SystemSpec("bulk", 1, n, True, box), cfg.model)
    check(gpu_lib, c2, pos, types, w, mode, what="box389")


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("T", [1, 5])
@pytest.mark.parametrize("dtype", [0, 1])
def test_interaction_block_counts(gpu_lib, dtype, T, mode):
    """One and five interaction blocks (fp32 and a bf16 filter) on four
    269-bead chains with biases."""
    import dataclasses
    cfg, pos, types, _ = make_config("cg269x64", n_replicas=4)
    m = dataclasses.replace(cfg.model, T=T, filter_dtype=dtype)
    w = make_weights(m, 4, bias_scale=0.05)
    check(gpu_lib, Config(f"chains-T{T}", cfg.system, m), pos, types, w, mode, n_replicas=4,
          what=f"T={T} dtype={dtype}")


@pytest.mark.parametrize("mode", list(MODES))
def test_bf16_filter(gpu_lib, mode):
    cfg, pos, types, w = make_config("md1024", n_replicas=4)
    check(gpu_lib, cfg, pos, types, w, mode, n_replicas=4, what="bf16 filter, 4 x 269")


@pytest.mark.parametrize("mode", list(MODES))
def test_cg269x64_full(gpu_lib, mode):
    cfg, pos, types, w = make_config("cg269x64")
    check(gpu_lib, cfg, pos, types, w, mode, what="cg269x64")


@pytest.mark.parametrize("mode", list(MODES))
def test_bulk4k_full(gpu_lib, mode):
    cfg, pos, types, w = make_config("bulk4k")
    check(gpu_lib, cfg, pos, types, w, mode, what="bulk4k")


def test_sparse_receivers(gpu_lib):
    from tests.test_gpu_energy_forces import sparse_clusters
    cfg = CONFIGS["cg32"]
    pos, types = sparse_clusters()
    w = make_weights(cfg.model, 2, bias_scale=0.05)
    c2 = Config("sparse", SystemSpec("chain_walk", 1, len(pos), False), cfg.model)
    for mode in MODES:
        check(gpu_lib, c2, pos, types, w, mode, what="sparse clusters")


def test_isolated_atoms(gpu_lib):
    """No edges at all: every edge tensor is empty and the forces vanish."""
    cfg = CONFIGS["cg32"]
    w = make_weights(cfg.model, 0, bias_scale=0.1)
    pos = (np.arange(12, dtype=np.float32)[:, None] * np.float32(40.0)).repeat(3, 1)
    types = np.zeros(12, np.int32)
    c2 = Config("iso", SystemSpec("chain_walk", 12, 1, False), cfg.model)
    for mode in MODES:
        E, F = check(gpu_lib, c2, pos, types, w, mode, what="12 single-atom replicas")
        assert np.all(F == 0)


def test_segmented_is_deterministic_and_matches_fused(gpu_lib):
    """Without atomics the unfused pipeline is bitwise reproducible, and it
    agrees with the fused kernels far inside the oracle bar."""
    import torch
    cfg, pos, types, w = make_config("cg269x64", n_replicas=3)
    m = cfg.model
    system = lib_system(gpu_lib, cfg.system, 3)
    E1, F1, _, _, s1 = run_unfused(gpu_lib, m, system, pos, types, w, m.r_cut, 0)
    E2, F2, _, _, s2 = run_unfused(gpu_lib, m, system, pos, types, w, m.r_cut, 0)
    assert s1[0] == 0 and s2[0] == 0
    assert np.array_equal(E1, E2) and np.array_equal(F1, F2)
    from tests.test_gpu_energy_forces import run_gpu
    Ef, Ff, _, _ = run_gpu(gpu_lib, m, system, pos, types, w, m.r_cut)
    rms = np.sqrt(np.mean(Ff ** 2))
    assert np.max(np.abs(E1 - Ef) / np.abs(Ef)) < 2e-6
    assert np.max(np.abs(F1 - Ff)) < 2e-5 * rms


def test_capacity_overflow_reported(gpu_lib):
    """A capacity below the list's edge count: the kernels stay inside the
    edge tensors they were given and the status word says SN_ERR_CAPACITY."""
    cfg, pos, types, w = make_config("cg32", seed=0)
    m = cfg.model
    system = lib_system(gpu_lib, cfg.system)
    for flags in MODES.values():
        _, _, _, col, status = run_unfused(gpu_lib, m, system, pos, types, w, m.r_cut, flags,
                                           cap=100)
        assert len(col) > 100
        assert status[0] == gpu_lib.SN_ERR_CAPACITY and status[1] == len(col)


def test_w16a16_model_is_rejected(gpu_lib):
    import dataclasses
    import torch
    cfg, pos, types, w = make_config("cg32", seed=0)
    m = dataclasses.replace(cfg.model, filter_dtype=2)
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


def test_host_validation(gpu_lib):
    import torch
    cfg, pos, types, w = make_config("cg32", seed=0)
    m = cfg.model
    desc = lib_desc(gpu_lib, m)
    system = lib_system(gpu_lib, cfg.system)
    model = gpu_lib.sn_model_create(desc, w)
    try:
        p, rowptr, col, ne, _ = gpu_neighbors(gpu_lib, system, pos, m.r_cut)
        t = torch.from_numpy(types).cuda()
        energy = torch.empty(1, dtype=torch.float32, device="cuda")
        forces = torch.empty(p.numel(), dtype=torch.float32, device="cuda")
        need = gpu_lib.sn_unfused_workspace_size(desc, system, ne)
        assert need > gpu_lib.sn_workspace_size(desc, system)
        small = gpu_lib.Workspace(need - 256)
        with pytest.raises(gpu_lib.SnError) as ex:
            gpu_lib.sn_energy_forces_unfused(model, system, p, t, rowptr, col, ne, 0, energy,
                                             forces, small)
        assert ex.value.status == gpu_lib.SN_ERR_WORKSPACE
        ws = gpu_lib.Workspace(need)
        for flags, cap in ((2, ne), (0, 0)):
            with pytest.raises(gpu_lib.SnError) as ex:
                gpu_lib.sn_energy_forces_unfused(model, system, p, t, rowptr, col, cap, flags,
                                                 energy, forces, ws)
            assert ex.value.status == gpu_lib.SN_ERR_INVALID_ARG
    finally:
        gpu_lib.sn_model_destroy(model)
