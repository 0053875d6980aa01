"""GPU neighbour list vs the oracle: exact (bit-for-bit) rowptr and col."""
import numpy as np
import pytest

import oracle
from gen.configs import CONFIGS, make_config
from tests.gpu_helpers import gpu_neighbors, lib_system, open_system

pytestmark = pytest.mark.gpu


def _compare(lib, system, pos, r_list):
    p, rowptr, col, ne, ws = gpu_neighbors(lib, system, pos, r_list)
    rp_ref, col_ref = oracle.neighbor_list(pos, system.n_replicas, system.atoms_per_replica,
                                           bool(system.periodic), system.box, r_list)
    assert ne == len(col_ref)
    assert np.array_equal(rowptr.cpu().numpy(), rp_ref)
    assert np.array_equal(col[:ne].cpu().numpy(), col_ref)
    assert lib.sn_get_device_status(ws)[0] == 0
    return ne


@pytest.mark.parametrize("name", ["cg32", "cg269x64", "bulk4k", "bulk64k"])
def test_configs_exact(gpu_lib, name):
    cfg, pos, types, w = make_config(name)
    ne = _compare(gpu_lib, lib_system(gpu_lib, cfg.system), pos, cfg.model.r_cut)
    print(f"{name}: {ne} directed edges")


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_chain_replicas_with_skin_exact(gpu_lib, seed):
    cfg, pos, types, w = make_config("cg269x64", seed=seed, n_replicas=16)
    _compare(gpu_lib, lib_system(gpu_lib, cfg.system, 16), pos, cfg.model.r_cut + 1.0)


@pytest.mark.parametrize("box,n,r", [(12.0, 300, 3.7), (16.0, 700, 5.0), (10.0, 97, 5.0)])
def test_periodic_small_boxes_exact(gpu_lib, box, n, r):
    """Cell mode (>= 3 cells per axis) and all-pairs mode (fewer cells) on
    boxes with ragged atom counts."""
    rng = np.random.default_rng(n)
    pos = rng.uniform(0, box, (n, 3)).astype(np.float32)
    pos[pos >= np.float32(box)] = 0
    _compare(gpu_lib, gpu_lib.make_system(1, n, True, box), pos, r)


def test_periodic_replicas_exact(gpu_lib):
    rng = np.random.default_rng(11)
    box, n, R = 14.0, 150, 5
    pos = rng.uniform(0, box, (R * n, 3)).astype(np.float32)
    _compare(gpu_lib, gpu_lib.make_system(R, n, True, box), pos, 4.5)


def test_pairs_at_the_radius(gpu_lib):
    r = np.float32(5.0)
    inside = np.nextafter(r, np.float32(0))
    outside = np.nextafter(r, np.float32(10))
    pos = np.array([[0, 0, 0], [inside, 0, 0], [20, 0, 0], [20 + r, 0, 0],
                    [40, 0, 0], [40 + outside, 0, 0], [60, 60, 60]], dtype=np.float32)
    ne = _compare(gpu_lib, gpu_lib.make_system(1, 7, False, 0.0), pos, float(r))
    assert ne == 2


@pytest.mark.parametrize("shape", ["cube", "ball", "slab", "outlier", "lattice"])
def test_open_system_cell_list_exact(gpu_lib, shape):
    """A large open system takes the cell list over its bounding box (the
    grid set on the device, no wrap-around at its faces); the list must
    equal the oracle's bit for bit."""
    pos, r = open_system(shape)
    ne = _compare(gpu_lib, gpu_lib.make_system(1, len(pos), False, 0.0), pos, r)
    print(f"open {shape}: {len(pos)} atoms, {ne} directed edges")
    assert ne > 0


@pytest.mark.parametrize("layout", ["overlapping", "offset", "periodic"])
def test_large_replicas_cell_list_exact(gpu_lib, layout):
    """Several replicas of 8,192 atoms or more share one cell list (open: over
    the bounding box of all of them; periodic: the cube), the pair test
    keeping replicas apart; the list must equal the oracle's bit for bit."""
    rng = np.random.default_rng([11, 7])
    rho, r = 0.0612, 5.0
    if layout == "periodic":
        R, n = 2, 8192
        box = float(np.float32((n / rho) ** (1 / 3)))
        pos = rng.uniform(0.0, box, (R * n, 3)).astype(np.float32)
        pos[pos >= np.float32(box)] = 0
        system = gpu_lib.make_system(R, n, True, box)
    else:
        R, n = 3, 9000
        side = (n / rho) ** (1 / 3)
        pos = rng.uniform(0.0, side, (R, n, 3))
        if layout == "offset":      # replicas side by side, one partly overlapping the next
            pos += np.array([0.7 * side, 0.0, -0.3 * side])[None, None, :] * np.arange(R)[:, None, None]
        pos = pos.reshape(-1, 3).astype(np.float32)
        system = gpu_lib.make_system(R, n, False, 0.0)
    ne = _compare(gpu_lib, system, pos, r)
    print(f"{layout}: {R} x {n} atoms, {ne} directed edges")
    assert ne > 0


def test_isolated_atoms_give_empty_rows(gpu_lib):
    pos = (np.arange(30, dtype=np.float32)[:, None] * np.float32(50.0)).repeat(3, 1)
    ne = _compare(gpu_lib, gpu_lib.make_system(3, 10, False, 0.0), pos, 5.0)
    assert ne == 0


def test_capacity_overflow_reports_and_leaves_rows_empty(gpu_lib):
    import torch
    cfg, pos, types, w = make_config("cg32")
    system = gpu_lib.make_system(1, 32, False, 0.0)
    rp_ref, col_ref = oracle.neighbor_list(pos, 1, 32, False, 0.0, cfg.model.r_cut)
    cap = len(col_ref) - 1
    p, rowptr, col, ne, ws = gpu_neighbors(gpu_lib, system, pos, cfg.model.r_cut, capacity=cap)
    status, detail, _ = gpu_lib.sn_get_device_status(ws)
    assert status == gpu_lib.SN_ERR_CAPACITY and detail == len(col_ref) and ne == len(col_ref)
    assert torch.all(rowptr == 0)
    assert torch.all(col == -7), "col must not be written on overflow"
    # exact fit succeeds after a reset
    gpu_lib.sn_reset_device_status(ws)
    p, rowptr, col, ne, ws = gpu_neighbors(gpu_lib, system, pos, cfg.model.r_cut,
                                           capacity=len(col_ref), ws=ws)
    assert gpu_lib.sn_get_device_status(ws)[0] == 0
    assert np.array_equal(col[:ne].cpu().numpy(), col_ref)


@pytest.mark.parametrize("n", [32768, 32769])
def test_row_scan_either_side_of_one_launch(gpu_lib, n):
    """Row counts of up to 32,768 receivers are scanned in one launch, more in
    three: exact lists on both sides, and an overflow reported with empty rows
    on both."""
    import torch
    rng = np.random.default_rng(n)
    box = 48.0
    pos = rng.uniform(0, box, (n, 3)).astype(np.float32)
    pos[pos >= np.float32(box)] = 0
    system = gpu_lib.make_system(1, n, True, box)
    ne = _compare(gpu_lib, system, pos, 3.0)
    p, rowptr, col, ne2, ws = gpu_neighbors(gpu_lib, system, pos, 3.0, capacity=ne - 1)
    status, detail, _ = gpu_lib.sn_get_device_status(ws)
    assert status == gpu_lib.SN_ERR_CAPACITY and detail == ne and ne2 == ne
    assert torch.all(rowptr == 0)


def test_host_validation(gpu_lib):
    import torch
    system = gpu_lib.make_system(1, 10, True, 9.0)
    pos = torch.zeros(30, device="cuda")
    rowptr = torch.zeros(11, dtype=torch.int32, device="cuda")
    col = torch.zeros(100, dtype=torch.int32, device="cuda")
    ws = gpu_lib.Workspace(gpu_lib.sn_workspace_size(None, system))
    with pytest.raises(gpu_lib.SnError) as e:
        gpu_lib.sn_build_neighbors(system, pos, 5.0, rowptr, col, 100, ws)   # box < 2 r
    assert e.value.status == gpu_lib.SN_ERR_INVALID_ARG
