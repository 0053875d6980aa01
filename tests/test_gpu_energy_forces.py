"""GPU energy and forces vs the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
from gen.configs import CONFIGS, ModelSpec, make_config, make_weights
from tests.gpu_helpers import (assert_energy_forces, gpu_neighbors, lib_desc, lib_system,
                               oracle_desc)

pytestmark = pytest.mark.gpu


def run_gpu(lib, m, system, pos, types, w, r_list, ws=None):
    import torch
    desc = lib_desc(lib, m)
    model = lib.sn_model_create(desc, w)
    try:
        if ws is None:
            ws = lib.Workspace(lib.sn_workspace_size(desc, system))
        p, rowptr, col, ne, ws = gpu_neighbors(lib, system, pos, r_list, ws=ws)
        t = torch.from_numpy(np.ascontiguousarray(types, dtype=np.int32)).cuda()
        energy = torch.empty(system.n_replicas, dtype=torch.float32, device="cuda")
        forces = torch.empty(p.numel(), dtype=torch.float32, device="cuda")
        lib.sn_energy_forces(model, system, p, t, rowptr, col, energy, forces, ws)
        torch.cuda.synchronize()
        status = lib.sn_get_device_status(ws)
        assert status[0] == 0, f"device status {status}"
        return (energy.cpu().double().numpy(), forces.cpu().double().numpy().reshape(-1, 3),
                rowptr.cpu().numpy(), col[:ne].cpu().numpy())
    finally:
        lib.sn_model_destroy(model)


def check(lib, cfg, pos, types, w, r_list=None, n_replicas=None, what=""):
    m = cfg.model
    system = lib_system(lib, cfg.system, n_replicas)
    r_list = m.r_cut if r_list is None else r_list
    E, F, rp, col = run_gpu(lib, m, system, pos, types, w, r_list)
    Eo, Fo = oracle.energy_forces(oracle_desc(m), w, pos, types, rp, col,
                                  n_replicas=system.n_replicas, periodic=bool(system.periodic),
                                  box=system.box)
    re, rf = assert_energy_forces(E, F, Eo, Fo, bf16=m.filter_dtype == 1, what=what)
    print(f"{what}: E rel {re:.2e}, F max/rms {rf:.2e}, edges {len(col)}")
    return E, F


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_cg32(gpu_lib, seed):
    cfg, pos, types, w = make_config("cg32", seed=seed)
    check(gpu_lib, cfg, pos, types, w, what=f"cg32 seed {seed}")


def test_cg32_with_biases_and_skin_list(gpu_lib):
    """Nonzero biases everywhere and a list built 1.5 A beyond the cutoff:
    listed edges at or beyond the cutoff must contribute nothing."""
    cfg, pos, types, w = make_config("cg32", seed=4, bias_scale=0.1)
    check(gpu_lib, cfg, pos, types, w, r_list=cfg.model.r_cut + 1.5, what="cg32 bias+skin")


def test_cg269_four_replicas(gpu_lib):
    cfg, pos, types, w = make_config("cg269x64", n_replicas=4, bias_scale=0.05)
    check(gpu_lib, cfg, pos, types, w, n_replicas=4, what="cg269x4")


def test_cg269x64_full(gpu_lib):
    cfg, pos, types, w = make_config("cg269x64")
    check(gpu_lib, cfg, pos, types, w, what="cg269x64")


def test_bulk4k_full(gpu_lib):
    cfg, pos, types, w = make_config("bulk4k")
    check(gpu_lib, cfg, pos, types, w, what="bulk4k")


def test_small_periodic_box_ragged(gpu_lib):
    """A periodic box whose atom count is not a multiple of any tile size."""
    cfg = CONFIGS["bulk4k"]
    rng = np.random.default_rng(3)
    n, box = 389, 17.9
    pos = rng.uniform(0, box, (n, 3)).astype(np.float32)
    pos[pos >= np.float32(box)] = 0
    types = rng.integers(0, 4, n).astype(np.int32)
    w = make_weights(cfg.model, 5, bias_scale=0.05)
    from gen.configs import Config, SystemSpec
    c2 = Config("box389", SystemSpec("bulk", 1, n, True, box), cfg.model)
    check(gpu_lib, c2, pos, types, w, what="box389")


def test_isolated_atoms_and_single_atom(gpu_lib):
    cfg = CONFIGS["cg32"]
    w = make_weights(cfg.model, 0, bias_scale=0.1)
    pos = (np.arange(12, dtype=np.float32)[:, None] * np.float32(40.0)).repeat(3, 1)
    types = np.zeros(12, np.int32)
    from gen.configs import Config, SystemSpec
    c2 = Config("iso", SystemSpec("chain_walk", 12, 1, False), cfg.model)
    E, F = check(gpu_lib, c2, pos, types, w, what="12 single-atom replicas")
    assert np.all(F == 0)


def test_bf16_filter(gpu_lib):
    cfg, pos, types, w = make_config("md1024", n_replicas=4)
    check(gpu_lib, cfg, pos, types, w, n_replicas=4, what="bf16 filter, 4 x 269")


def test_deterministic_and_batched_equals_single(gpu_lib):
    import torch
    cfg, pos, types, w = make_config("cg269x64", n_replicas=3)
    m = cfg.model
    sys3 = lib_system(gpu_lib, cfg.system, 3)
    E1, F1, _, _ = run_gpu(gpu_lib, m, sys3, pos, types, w, m.r_cut)
    E2, F2, _, _ = run_gpu(gpu_lib, m, sys3, pos, types, w, m.r_cut)
    assert np.array_equal(E1, E2) and np.array_equal(F1, F2), "run-to-run results differ"
    for r in range(3):
        sl = slice(r * 269, (r + 1) * 269)
        Er, Fr, _, _ = run_gpu(gpu_lib, m, lib_system(gpu_lib, cfg.system, 1), pos[sl], types[sl], w,
                               m.r_cut)
        assert abs(Er[0] - E1[r]) <= 1e-6 * abs(E1[r])
        assert np.max(np.abs(Fr - F1[sl])) <= 1e-5 * np.sqrt(np.mean(F1[sl] ** 2))


def test_net_force_and_translation(gpu_lib):
    cfg, pos, types, w = make_config("bulk4k")
    m = cfg.model
    system = lib_system(gpu_lib, cfg.system)
    E, F, _, _ = run_gpu(gpu_lib, m, system, pos, types, w, m.r_cut)
    rms = np.sqrt(np.mean(F ** 2))
    assert np.max(np.abs(F.sum(axis=0))) < 1e-3 * rms * np.sqrt(len(F))
