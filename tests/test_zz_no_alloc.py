"""sn_energy_forces_noalloc (the library's static device workspace, for
callers that cannot allocate) against sn_energy_forces with a workspace of
the caller's, through the C ABI: the same kernels on the same inputs, so
the energies and forces must agree bit for bit (and therefore also meet the
oracle's bars, checked too). Two calls in a row, the second on a smaller
system with another model, so the second runs on the array the first left
behind; then a system too large for the array is refused, and an error
found on the device is reported through status_dev."""
import numpy as np
import pytest

import oracle
from gen.configs import make_config
from tests.gpu_helpers import (assert_energy_forces, gpu_neighbors, lib_desc, lib_system,
                               oracle_desc, oracle_list)

pytestmark = pytest.mark.gpu


def _both(lib, cfg, pos, types, w):
    import torch
    m = cfg.model
    system = lib_system(lib, cfg.system)
    desc = lib_desc(lib, m)
    assert lib.sn_workspace_size(desc, system) <= lib.SN_SCRATCH_BYTES
    model = lib.sn_model_create(desc, w)
    try:
        p, rowptr, col, ne, _ = gpu_neighbors(lib, system, pos, m.r_cut)
        t = torch.from_numpy(np.ascontiguousarray(types, dtype=np.int32)).cuda()
        n = system.n_replicas * system.atoms_per_replica
        e_ref = torch.empty(system.n_replicas, dtype=torch.float32, device="cuda")
        f_ref = torch.empty(3 * n, dtype=torch.float32, device="cuda")
        ws = lib.Workspace(lib.sn_workspace_size(desc, system))
        lib.sn_energy_forces(model, system, p, t, rowptr, col, e_ref, f_ref, ws)
        e_na = torch.full_like(e_ref, float("nan"))
        f_na = torch.full_like(f_ref, float("nan"))
        st = torch.full((2,), -5, dtype=torch.int64, device="cuda")
        lib.sn_energy_forces_noalloc(model, system, p, t, rowptr, col, e_na, f_na, st)
        torch.cuda.synchronize()
        assert lib.sn_get_device_status(ws)[0] == 0
        assert st.cpu().tolist() == [0, 0]
        assert torch.equal(e_na, e_ref) and torch.equal(f_na, f_ref)
        E = e_na.cpu().double().numpy()
        F = f_na.cpu().double().numpy().reshape(-1, 3)
        rp, cl = oracle_list(system, pos, m.r_cut, rowptr.cpu().numpy(), col[:ne].cpu().numpy())
        Eo, Fo, eps = oracle.energy_forces(oracle_desc(m), w, pos, types, rp, cl,
                                           n_replicas=system.n_replicas,
                                           periodic=bool(system.periodic), box=system.box,
                                           return_eps=True)
        assert_energy_forces(E, F, Eo, Fo, bf16=m.filter_dtype in (1, 2),
                             eps_abs_sum=np.abs(eps).reshape(system.n_replicas, -1).sum(axis=1),
                             w16=m.filter_dtype == 2)
    finally:
        lib.sn_model_destroy(model)


def test_noalloc_matches_workspace_call_twice(gpu_lib):
    cfg, pos, types, w = make_config("bulk4k")
    _both(gpu_lib, cfg, pos, types, w)
    cfg, pos, types, w = make_config("cg32", seed=1, bias_scale=0.05)
    _both(gpu_lib, cfg, pos, types, w)


def test_noalloc_refuses_large_systems_and_reports_device_errors(gpu_lib):
    import torch
    lib = gpu_lib
    cfg, pos, types, w = make_config("cg269x64")
    m = cfg.model
    system = lib_system(lib, cfg.system)
    desc = lib_desc(lib, m)
    assert lib.sn_workspace_size(desc, system) > lib.SN_SCRATCH_BYTES
    model = lib.sn_model_create(desc, w)
    try:
        n = system.n_replicas * system.atoms_per_replica
        p, rowptr, col, ne, _ = gpu_neighbors(lib, system, pos, m.r_cut)
        t = torch.from_numpy(types).cuda()
        e = torch.empty(system.n_replicas, dtype=torch.float32, device="cuda")
        f = torch.empty(3 * n, dtype=torch.float32, device="cuda")
        st = torch.zeros(2, dtype=torch.int64, device="cuda")
        with pytest.raises(lib.SnError) as err:
            lib.sn_energy_forces_noalloc(model, system, p, t, rowptr, col, e, f, st)
        assert err.value.status == lib.SN_ERR_WORKSPACE
    finally:
        lib.sn_model_destroy(model)
    # a type out of range is found on the device and reported with its atom
    cfg, pos, types, w = make_config("cg32")
    m = cfg.model
    system = lib_system(lib, cfg.system)
    model = lib.sn_model_create(lib_desc(lib, m), w)
    try:
        p, rowptr, col, ne, _ = gpu_neighbors(lib, system, pos, m.r_cut)
        bad = types.copy()
        bad[7] = m.n_types + 3
        t = torch.from_numpy(bad).cuda()
        e = torch.empty(1, dtype=torch.float32, device="cuda")
        f = torch.empty(96, dtype=torch.float32, device="cuda")
        st = torch.zeros(2, dtype=torch.int64, device="cuda")
        lib.sn_energy_forces_noalloc(model, system, p, t, rowptr, col, e, f, st)
        torch.cuda.synchronize()
        assert st.cpu().tolist() == [lib.SN_ERR_INVALID_ARG, 7]
        # and the next call starts from a clear status again
        t = torch.from_numpy(types).cuda()
        lib.sn_energy_forces_noalloc(model, system, p, t, rowptr, col, e, f, st)
        torch.cuda.synchronize()
        assert st.cpu().tolist() == [0, 0]
    finally:
        lib.sn_model_destroy(model)
