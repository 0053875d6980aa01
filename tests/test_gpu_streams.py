"""The C ABI on the caller's streams: every call enqueues its work on the stream
it is given, a model serves several streams at once, and a workspace belongs
to one stream. Results on side streams must equal those on the default
stream bit for bit (the path has no atomics and a fixed summation order)."""
import numpy as np
import pytest

from gen.configs import make_config
from tests.gpu_helpers import gpu_neighbors, lib_desc, lib_system

pytestmark = pytest.mark.gpu


def test_two_streams_share_a_model(gpu_lib):
    import torch
    lib = gpu_lib
    cfg, pos, types, w = make_config("cg269x64", n_replicas=8)
    m = cfg.model
    system = lib_system(lib, cfg.system, 8)
    desc = lib_desc(lib, m)
    n = 8 * cfg.system.atoms_per_replica
    model = lib.sn_model_create(desc, w)
    try:
        size = lib.sn_workspace_size(desc, system)
        ws0 = lib.Workspace(size)
        p, rowptr, col, ne, ws0 = gpu_neighbors(lib, system, pos, m.r_cut, ws=ws0)
        t = torch.from_numpy(np.ascontiguousarray(types, dtype=np.int32)).cuda()
        E0 = torch.empty(8, dtype=torch.float32, device="cuda")
        F0 = torch.empty(3 * n, dtype=torch.float32, device="cuda")
        lib.sn_energy_forces(model, system, p, t, rowptr, col, E0, F0, ws0)
        torch.cuda.synchronize()
        # two side streams (default priority), each with its own workspace,
        # list and outputs, allocated and cleared before the streams start
        sides = []
        for _ in range(2):
            ws = lib.Workspace(size)
            rp = torch.full((n + 1,), -1, dtype=torch.int32, device="cuda")
            cl = torch.full((ne,), -1, dtype=torch.int32, device="cuda")
            E = torch.full((8,), float("nan"), dtype=torch.float32, device="cuda")
            F = torch.full((3 * n,), float("nan"), dtype=torch.float32, device="cuda")
            sides.append((torch.cuda.Stream(), ws, rp, cl, E, F))
        torch.cuda.synchronize()
        for s, ws, rp, cl, E, F in sides:
            with torch.cuda.stream(s):
                lib.sn_build_neighbors(system, p, m.r_cut, rp, cl, ne, ws, return_count=False)
                for _ in range(3):
                    lib.sn_energy_forces(model, system, p, t, rp, cl, E, F, ws)
        torch.cuda.synchronize()
        for s, ws, rp, cl, E, F in sides:
            assert lib.sn_get_device_status(ws)[0] == 0
            assert torch.equal(rp, rowptr) and torch.equal(cl, col[:ne])
            assert torch.equal(E, E0) and torch.equal(F, F0)
    finally:
        lib.sn_model_destroy(model)


def test_md_on_a_side_stream(gpu_lib):
    """Initialisation and eight BAOAB steps (a scheduled rebuild included) on a
    side stream give the default stream's state bit for bit."""
    import torch
    lib = gpu_lib
    cfg, pos, types, w = make_config("cg269x64", n_replicas=3)
    m = cfg.model
    system = lib_system(lib, cfg.system, 3)
    desc = lib_desc(lib, m)
    model = lib.sn_model_create(desc, w)
    try:
        size = lib.sn_workspace_size(desc, system)
        t = torch.from_numpy(np.ascontiguousarray(types, dtype=np.int32)).cuda()
        params = lib.make_md_params(2.0, 300.0, 1.0, 100.0, 1.0, 5, 7)
        runs = []
        for side in (False, True):
            p = torch.from_numpy(pos).cuda().reshape(-1)
            state = lib.MdState(p, 400 * len(pos), active=True)
            energy = torch.empty(3, dtype=torch.float32, device="cuda")
            ws = lib.Workspace(size)
            s = torch.cuda.Stream() if side else torch.cuda.current_stream()
            torch.cuda.synchronize()
            with torch.cuda.stream(s):
                lib.sn_md_init(model, system, t, params, state, energy, ws)
                lib.sn_md_step(model, system, t, params, state, 8, energy, ws)
            torch.cuda.synchronize()
            assert lib.sn_get_device_status(ws)[0] == 0
            runs.append((state.pos.clone(), state.vel.clone(), state.forces.clone(),
                         energy.clone()))
        for a, b in zip(*runs):
            assert torch.equal(a, b)
    finally:
        lib.sn_model_destroy(model)
