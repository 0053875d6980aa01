"""GPU energy and forces vs the fp64 oracle, through the C ABI."""
import numpy as np
import pytest

import oracle
from gen.configs import CONFIGS, ModelSpec, make_config, make_weights
from tests.gpu_helpers import (assert_energy_forces, cutout_forces, depth_scale, gpu_neighbors,
                               lib_desc, lib_system, oracle_desc, oracle_list, F_TOL_BF16,
                               F_TOL_F32, F_TOL_W16)

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
    E, F, rp_gpu, col_gpu = run_gpu(lib, m, system, pos, types, w, r_list)
    rp, col = oracle_list(system, pos, r_list, rp_gpu, col_gpu, what)
    Eo, Fo, eps = oracle.energy_forces(oracle_desc(m), w, pos, types, rp, col,
                                       n_replicas=system.n_replicas,
                                       periodic=bool(system.periodic), box=system.box,
                                       return_eps=True)
    eps_sum = np.abs(eps).reshape(system.n_replicas, -1).sum(axis=1)
    re, rf = assert_energy_forces(E, F, Eo, Fo, bf16=m.filter_dtype in (1, 2), what=what,
                                  eps_abs_sum=eps_sum, w16=m.filter_dtype == 2,
                                  depth=depth_scale(m.T))
    if m.filter_dtype in (1, 2):
        print(f"{what}: E err / sum|eps| {np.max(np.abs(E - Eo) / eps_sum):.2e}")
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


@pytest.mark.parametrize("T", [1, 5])
@pytest.mark.parametrize("dtype", [0, 1, 2, 3])
def test_interaction_block_counts(gpu_lib, T, dtype):
    """One interaction block (only the first block's backward kernel, on its
    own worker partition, and the force sum over one block) and five (three
    blocks with source sums between the first and the last), at fp32, with a
    bf16 filter, W16A16 and fp32 on fp16 pairs, on four 269-bead chains with
    biases."""
    import dataclasses
    from gen.configs import Config
    cfg, pos, types, _ = make_config("cg269x64", n_replicas=4)
    m = dataclasses.replace(cfg.model, T=T, filter_dtype=dtype)
    w = make_weights(m, 4, bias_scale=0.05)
    c2 = Config(f"chains-T{T}", cfg.system, m)
    check(gpu_lib, c2, pos, types, w, n_replicas=4, what=f"T={T} dtype={dtype}")


# Model shapes the API accepts beyond the workloads' (D, Dr, T, H): a basis of
# two functions and of one past a 32-wide chunk, a 32-wide readout at D 128,
# a single block and the largest block count.
SHAPES = [(64, 2, 1, 32), (64, 33, 2, 64), (128, 7, 2, 32), (128, 31, 1, 64), (128, 63, 8, 64)]


@pytest.mark.parametrize("dtype", [0, 1, 2, 3])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "D%d-Dr%d-T%d-H%d" % s)
def test_model_shapes(gpu_lib, shape, dtype):
    """Each shape in every precision on four 269-bead chains with biases."""
    import dataclasses
    from gen.configs import Config
    D, Dr, T, H = shape
    cfg, pos, types, _ = make_config("cg269x64", n_replicas=4)
    m = dataclasses.replace(cfg.model, D=D, Dr=Dr, T=T, H=H, filter_dtype=dtype)
    w = make_weights(m, 11, bias_scale=0.05)
    check(gpu_lib, Config("shape", cfg.system, m), pos, types, w, n_replicas=4,
          what=f"D{D} Dr{Dr} T{T} H{H} dtype {dtype}")


def test_cg269x64_full(gpu_lib):
    cfg, pos, types, w = make_config("cg269x64")
    check(gpu_lib, cfg, pos, types, w, what="cg269x64")


def test_bulk4k_full(gpu_lib):
    cfg, pos, types, w = make_config("bulk4k")
    check(gpu_lib, cfg, pos, types, w, what="bulk4k")


@pytest.mark.parametrize("factor", [0.4, 0.6])
def test_compact_chains_long_rows(gpu_lib, factor):
    """Chains compacted about their centroids: receiver rows of up to ~170
    edges span many tiles, and most contacts are sequence-distant."""
    from gen.systems import rescale_replicas
    cfg, pos, types, w = make_config("cg269x64", n_replicas=4, bias_scale=0.05)
    pos = rescale_replicas(pos, 269, factor)
    check(gpu_lib, cfg, pos, types, w, n_replicas=4, what=f"cg269x4 compacted x{factor}")


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


def test_open_cluster_cell_list(gpu_lib):
    """Energies and forces of a large open cluster (a ball of 16,384 atoms at
    the bulk density, the bulk model with biases), whose list the library
    builds from cells over the bounding box, against the oracle."""
    from gen.configs import Config, SystemSpec
    from tests.gpu_helpers import open_system
    cfg = CONFIGS["bulk4k"]
    pos, r = open_system("ball", seed=9)
    n = len(pos)
    types = np.random.default_rng(12).integers(0, 4, n).astype(np.int32)
    w = make_weights(cfg.model, 6, bias_scale=0.05)
    c2 = Config("ball16k", SystemSpec("bulk", 1, n, False, 0.0), cfg.model)
    check(gpu_lib, c2, pos, types, w, r_list=cfg.model.r_cut, what="open ball")


def sparse_clusters(n_iso=100, seed=11):
    """Clusters of 10 atoms (index-contiguous, 4 A apart on a helix) separated
    in index order by runs of isolated atoms 50 A apart: one 16-edge tile
    then spans receivers more than 64 apart, most of them without edges."""
    rng = np.random.default_rng(seed)
    pos, types = [], []
    for c in range(4):
        base = np.array([0.0, 0.0, 400.0 * c])
        for k in range(10):
            ang = 1.7 * k
            pos.append(base + [3.0 * np.cos(ang), 3.0 * np.sin(ang), 1.5 * k])
            types.append(0)
        for k in range(n_iso if c < 3 else 7):
            pos.append(base + [60.0 + 50.0 * k, 0.0, 0.0])
            types.append(0)
    pos = np.asarray(pos, np.float32) + rng.normal(0, 0.05, (len(pos), 3)).astype(np.float32)
    return pos, np.asarray(types, np.int32)


def test_sparse_receivers_beyond_the_window(gpu_lib):
    """1200 replicas of the sparse pattern: every worker owns ~100 receivers
    or more, so tiles cross runs of >64 edgeless receivers (the segment-end
    window's fallback path)."""
    from gen.configs import Config, SystemSpec
    cfg = CONFIGS["cg32"]
    pos, types = sparse_clusters()
    R = 1200
    w = make_weights(cfg.model, 2, bias_scale=0.05)
    c2 = Config("sparse", SystemSpec("chain_walk", R, len(pos), False), cfg.model)
    check(gpu_lib, c2, np.tile(pos, (R, 1)), np.tile(types, R), w, n_replicas=R,
          what="sparse clusters x1200")


@pytest.mark.parametrize("dtype", [0, 1, 2, 3])
def test_coincident_atoms(gpu_lib, dtype):
    """Pairs at distance zero (a bead moved onto its bonded neighbour, and two
    beads far apart in sequence made to coincide): the energy is defined,
    and the pair's force term, whose direction u / d is undefined there, is
    zero on both sides (the oracle divides by 1 where d = 0, the kernels
    take 1 / d as 0)."""
    import dataclasses
    from gen.configs import Config
    cfg, pos, types, _ = make_config("cg269x64", n_replicas=4)
    pos = pos.copy()
    pos[5] = pos[6]
    pos[269 + 100] = pos[269 + 200]
    m = dataclasses.replace(cfg.model, filter_dtype=dtype)
    w = make_weights(m, 4, bias_scale=0.05)
    check(gpu_lib, Config("coincident", cfg.system, m), pos, types, w, n_replicas=4,
          what=f"coincident beads dtype {dtype}")


def test_out_of_range_types_reported(gpu_lib):
    """An atom type outside [0, n_types) is reported in the device status
    word (SN_ERR_INVALID_ARG, detail = an offending atom) instead of being
    read past the embedding table (the set-up kernel clamps it to 0)."""
    import torch
    cfg, pos, types, w = make_config("cg269x64", n_replicas=2)
    m = cfg.model
    system = lib_system(gpu_lib, cfg.system, 2)
    bad = types.copy()
    bad[17] = m.n_types
    bad[300] = -1
    desc = lib_desc(gpu_lib, m)
    model = gpu_lib.sn_model_create(desc, w)
    try:
        ws = gpu_lib.Workspace(gpu_lib.sn_workspace_size(desc, system))
        p, rowptr, col, ne, ws = gpu_neighbors(gpu_lib, system, pos, m.r_cut, ws=ws)
        t = torch.from_numpy(np.ascontiguousarray(bad, dtype=np.int32)).cuda()
        n = 2 * cfg.system.atoms_per_replica
        energy = torch.empty(2, dtype=torch.float32, device="cuda")
        forces = torch.empty(3 * n, dtype=torch.float32, device="cuda")
        gpu_lib.sn_energy_forces(model, system, p, t, rowptr, col, energy, forces, ws)
        torch.cuda.synchronize()
        status, detail, _ = gpu_lib.sn_get_device_status(ws)
        assert status == gpu_lib.SN_ERR_INVALID_ARG and detail in (17, 300), (status, detail)
    finally:
        gpu_lib.sn_model_destroy(model)


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


def _w16a16(cfg):
    import dataclasses
    return dataclasses.replace(cfg, model=dataclasses.replace(cfg.model, filter_dtype=2))


@pytest.mark.parametrize("dtype", [1, 2])
def test_16bit_small_model(gpu_lib, dtype):
    """The D 64 / Dr 32 / H 32 model with a bf16 filter (one 32-wide basis
    chunk) or W16A16, on a chain with biases."""
    import dataclasses
    cfg, pos, types, w = make_config("cg32", seed=3, bias_scale=0.05)
    c2 = dataclasses.replace(cfg, model=dataclasses.replace(cfg.model, filter_dtype=dtype))
    check(gpu_lib, c2, pos, types, w, what=f"cg32 filter_dtype {dtype}")


def test_bf16_periodic_box(gpu_lib):
    import dataclasses
    cfg = CONFIGS["bulk4k"]
    rng = np.random.default_rng(4)
    n, box = 389, 17.9
    pos = rng.uniform(0, box, (n, 3)).astype(np.float32)
    pos[pos >= np.float32(box)] = 0
    types = rng.integers(0, 4, n).astype(np.int32)
    w = make_weights(cfg.model, 6, bias_scale=0.05)
    from gen.configs import Config, SystemSpec
    c2 = Config("box389", SystemSpec("bulk", 1, n, True, box),
                dataclasses.replace(cfg.model, filter_dtype=1))
    check(gpu_lib, c2, pos, types, w, what="bf16 box389")


@pytest.mark.parametrize("name,nrep", [("md1024", 4), ("cg32", None)])
def test_w16a16_chains(gpu_lib, name, nrep):
    """fp16 operands with per-channel scales in every MLP (D 128 / H 64 and
    D 64 / H 32 shapes) against the oracle with the same quantized weights."""
    cfg, pos, types, w = make_config(name, n_replicas=nrep, bias_scale=0.05)
    check(gpu_lib, _w16a16(cfg), pos, types, w, n_replicas=nrep, what=f"W16A16 {name}")


def test_w16a16_periodic_box(gpu_lib):
    cfg = CONFIGS["bulk4k"]
    rng = np.random.default_rng(3)
    n, box = 389, 17.9
    pos = rng.uniform(0, box, (n, 3)).astype(np.float32)
    pos[pos >= np.float32(box)] = 0
    types = rng.integers(0, 4, n).astype(np.int32)
    w = make_weights(cfg.model, 5, bias_scale=0.05)
    from gen.configs import Config, SystemSpec
    c2 = Config("box389", SystemSpec("bulk", 1, n, True, box), cfg.model)
    check(gpu_lib, _w16a16(c2), pos, types, w, what="W16A16 box389")


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


def test_md1024_full_sampled_replicas(gpu_lib):
    """All 1024 replicas of the bf16 MD workload on the GPU; replicas are
    independent, so sampled ones are checked exactly against the oracle run
    on that replica alone."""
    cfg, pos, types, w = make_config("md1024")
    m = cfg.model
    system = lib_system(gpu_lib, cfg.system)
    E, F, _, _ = run_gpu(gpu_lib, m, system, pos, types, w, m.r_cut)
    n = cfg.system.atoms_per_replica
    for r in (0, 377, 1023):
        sl = slice(r * n, (r + 1) * n)
        rp, col = oracle.neighbor_list(pos[sl], 1, n, False, 0.0, m.r_cut)
        Eo, Fo, eps = oracle.energy_forces(oracle_desc(m), w, pos[sl], types[sl], rp, col,
                                           n_replicas=1, periodic=False, box=0.0, return_eps=True)
        re, rf = assert_energy_forces(E[r:r + 1], F[sl], Eo, Fo, bf16=True, what=f"md1024 r{r}",
                                      eps_abs_sum=[np.abs(eps).sum()])
        print(f"md1024 replica {r}: E rel {re:.2e}, F max/rms {rf:.2e}")


def test_bulk4k_tiled_2x2x2(gpu_lib):
    """The bulk4k system repeated 2 x 2 x 2 in a box of twice the side (32,768
    atoms, the large-system cell-list path): with r_c below half the small box
    every copy sees the same environment, so the energy is 8x and the forces
    repeat those of the oracle on the small box. Positions sit on a 2^-12 A
    grid and the side is 40.625 A, so every shifted coordinate is exact in
    fp32 and all copies have the same geometry."""
    cfg, pos, types, w = make_config("bulk4k")
    m = cfg.model
    L = np.float32(40.625)
    q = np.float32(2.0 ** -12)
    pos = (np.floor(pos.astype(np.float64) * (float(L) / cfg.system.box) / float(q)) * float(q))
    pos = np.mod(pos, float(L)).astype(np.float32)
    shifts = np.array([(a, b, c) for a in (0, 1) for b in (0, 1) for c in (0, 1)], np.float32) * L
    big = np.concatenate([pos + s for s in shifts]).astype(np.float32)
    assert np.array_equal(big[4096:8192] - shifts[1], pos)      # shifts are exact
    big_types = np.tile(types, 8)
    from gen.configs import Config, SystemSpec
    c2 = Config("bulk4k_x8", SystemSpec("bulk", 1, len(big), True, float(2 * L)), m)
    system = lib_system(gpu_lib, c2.system)
    E, F, _, col = run_gpu(gpu_lib, m, system, big, big_types, w, m.r_cut)
    rp, c4 = oracle.neighbor_list(pos, 1, len(pos), True, float(L), m.r_cut)
    assert len(col) == 8 * len(c4)
    Eo, Fo = oracle.energy_forces(oracle_desc(m), w, pos, types, rp, c4, n_replicas=1,
                                  periodic=True, box=float(L))
    re, rf = assert_energy_forces(E, F, 8 * Eo, np.tile(Fo, (8, 1)), what="bulk4k x8")
    print(f"bulk4k x8: E rel {re:.2e}, F max/rms {rf:.2e}")


def test_bulk64k_full_invariances(gpu_lib):
    """The 65,536-atom box at full size: a periodic translation leaves energy
    and forces unchanged and the net force vanishes. Positions sit on a
    2^-10 A grid, the side (102.25 A) and the shift on a 1/4 A grid, so the
    translated and wrapped coordinates are exact in fp32 and only the
    kernels' own rounding (their order of summation over receivers and
    tiles changes with the atom order in space) separates the two runs."""
    cfg, pos, types, w = make_config("bulk64k")
    m = cfg.model
    L = 102.25
    q = 2.0 ** -10
    pos = np.mod(np.floor(pos.astype(np.float64) * (L / cfg.system.box) / q) * q, L)
    pos = pos.astype(np.float32)
    from gen.configs import Config, SystemSpec
    c2 = Config("bulk64k_grid", SystemSpec("bulk", 1, len(pos), True, L), m)
    system = lib_system(gpu_lib, c2.system)
    E, F, _, _ = run_gpu(gpu_lib, m, system, pos, types, w, m.r_cut)
    shift = np.array([16.25, -5.0, 40.75])
    moved = np.mod(pos.astype(np.float64) + shift, L)
    assert np.all(moved == moved.astype(np.float32))               # exact in fp32
    E2, F2, _, _ = run_gpu(gpu_lib, m, system, moved.astype(np.float32), types, w, m.r_cut)
    rms = np.sqrt(np.mean(F ** 2))
    assert abs(E2[0] - E[0]) <= 1e-5 * abs(E[0]), (E, E2)
    assert np.max(np.abs(F2 - F)) <= 1e-4 * rms, np.max(np.abs(F2 - F)) / rms
    assert np.max(np.abs(F.sum(axis=0))) < 1e-3 * rms * np.sqrt(len(F))


def test_bulk64k_full_vs_oracle(gpu_lib):
    """The 65,536-atom box at full size, in the bench's launch configuration,
    against the oracle's values stored by tests/golden/make_bulk64k.py (the
    oracle's own list of 2.1M edges; minutes of host time, so computed once):
    the total energy, and the forces on the atoms within 6 A of four centre
    atoms spread over the box, element by element (from exact cutouts). fp32
    weights (the fp32 filter and the fp32 model on fp16 pairs) at the fp32
    bars, the bf16 filter and W16A16 at their 16-bit bars."""
    import dataclasses
    import json
    import os
    from tests.gpu_helpers import E_TOL_BF16_ABS_SUM, E_TOL_F32, E_TOL_W16_ABS_SUM
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                       "bulk64k_oracle.json")))
    cfg, pos, types, w = make_config("bulk64k")
    m = cfg.model
    system = lib_system(gpu_lib, cfg.system)
    for dtype in (0, 3, 1, 2):
        ref = str(0 if dtype == 3 else dtype)
        E, F, _, col = run_gpu(gpu_lib, dataclasses.replace(m, filter_dtype=dtype), system, pos,
                               types, w, m.r_cut)
        assert len(col) == gold["edges"]
        Eo = gold["energy"][ref]["E"]
        atoms = np.asarray(gold["forces"][ref]["atoms"])
        Fo = np.asarray(gold["forces"][ref]["F"])
        rms = np.sqrt(np.mean(Fo ** 2))
        ferr = np.max(np.abs(F[atoms] - Fo)) / rms
        if dtype in (1, 2):
            eerr = abs(E[0] - Eo) / gold["energy"][ref]["sum_abs_eps"]
            ebar = E_TOL_W16_ABS_SUM if dtype == 2 else E_TOL_BF16_ABS_SUM
        else:
            eerr = abs(E[0] - Eo) / abs(Eo)
            ebar = E_TOL_F32
        print(f"bulk64k dtype {dtype}: E {E[0]:.6f} vs {Eo:.6f} (err {eerr:.2e}), "
              f"{len(atoms)} atoms F max/rms {ferr:.2e}")
        assert eerr <= ebar
        assert ferr <= (F_TOL_F32 if dtype in (0, 3) else F_TOL_BF16 if dtype == 1 else F_TOL_W16)


@pytest.mark.parametrize("dtype", [0, 1, 2, 3])
def test_small_and_large_batches_agree(gpu_lib, dtype):
    """With fp32 atom-wise operands (the fp32 filter) and up to two 16-atom
    tiles per SIMD, the atom-wise networks run with four waves per tile (each
    a quarter of the hidden and output features), above that with one. The
    first 8 replicas of a 160-replica batch of the MD model's chains (2,690
    tiles) against the same 8 alone (135 tiles): same energies and forces
    within the fp32 bars (1e-5 relative, 1e-4 of the force RMS); for the
    bf16 filter and fp16 pairs (atom-wise layers on fp16 pairs) and W16A16
    (within its own bars: an fp32 rounding difference in a feature can move
    one of its fp16 roundings), which take one wave per tile at both sizes,
    a check of size invariance alone."""
    import dataclasses
    cfg, pos, types, w = make_config("md1024", n_replicas=160)
    m = dataclasses.replace(cfg.model, filter_dtype=dtype)
    nper = cfg.system.atoms_per_replica
    E1, F1, _, _ = run_gpu(gpu_lib, m, lib_system(gpu_lib, cfg.system, 160), pos, types, w,
                           m.r_cut)
    k = 8 * nper
    E2, F2, _, _ = run_gpu(gpu_lib, m, lib_system(gpu_lib, cfg.system, 8), pos[:k], types[:k], w,
                           m.r_cut)
    F1 = np.asarray(F1).reshape(-1, 3)[:k]
    F2 = np.asarray(F2).reshape(-1, 3)
    rms = np.sqrt(np.mean(F2 ** 2))
    de = np.max(np.abs(E1[:8] - E2) / np.abs(E2))
    df = np.max(np.abs(F1 - F2)) / rms
    print(f"dtype {dtype}: E rel {de:.2e}, F max/rms {df:.2e}")
    if dtype == 2:
        assert de <= 1e-4 and df <= F_TOL_W16
    else:
        assert de <= 1e-5 and df <= F_TOL_F32


@pytest.mark.parametrize("dtype", [0, 3])
def test_rows_cut_by_worker_boundaries(gpu_lib, dtype):
    """Workers take whole 16-edge tiles, so receiver rows are cut between
    workers, the other workers' parts added where the rows are read (the
    atom-wise kernels, the force sum): 16 mutually neighbouring atoms (rows
    of 15 against tiles of 16, one tile per worker) and 200 atoms in a 9 A
    ball at about bulk density (rows of ~120-199 edges spanning several
    workers), with biases."""
    import dataclasses
    from gen.configs import Config, SystemSpec
    cfg = CONFIGS["cg32"]
    m = dataclasses.replace(cfg.model, filter_dtype=dtype)
    rng = np.random.default_rng(21)
    w = make_weights(cfg.model, 8, bias_scale=0.05)
    for n, radius in ((16, 4.5), (200, 9.0)):
        d = rng.standard_normal((n, 3))
        d /= np.linalg.norm(d, axis=1, keepdims=True)
        pos = (d * radius * rng.uniform(0.2, 1.0, (n, 1)) ** (1 / 3)).astype(np.float32)
        types = np.zeros(n, np.int32)
        c2 = Config(f"ball{n}", SystemSpec("chain_walk", 1, n, False), m)
        check(gpu_lib, c2, pos, types, w, what=f"ball of {n}, dtype {dtype}")


def test_readout_as_wide_as_the_features(gpu_lib):
    """D 64 with a readout hidden width H 64 (H == D): the readout runs the
    same kernel shape as the update networks; every precision."""
    import dataclasses
    cfg, pos, types, _ = make_config("cg32", seed=5)
    for dtype in (0, 1, 2, 3):
        m = dataclasses.replace(cfg.model, H=64, filter_dtype=dtype)
        w = make_weights(m, 9, bias_scale=0.05)
        check(gpu_lib, dataclasses.replace(cfg, model=m), pos, types, w,
              what=f"cg32 D 64 H 64 dtype {dtype}")


def test_bulk64k_relabelled_in_cell_order(gpu_lib):
    """The same 65,536-atom box with its atoms relabelled in the order of 5 A
    cells (the order a cell-sorted MD code keeps; bench.py --order cell):
    the list, the tile partition and every summation order change, the
    energy and the relabelled forces must not. Against the stored oracle
    values, fp32 bars."""
    import json
    import os
    from gen.systems import cell_order
    from tests.gpu_helpers import E_TOL_F32
    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden",
                                       "bulk64k_oracle.json")))
    cfg, pos, types, w = make_config("bulk64k")
    m = cfg.model
    k = cell_order(pos, cfg.system.box)
    inv = np.empty_like(k)
    inv[k] = np.arange(len(k))
    system = lib_system(gpu_lib, cfg.system)
    E, F, _, col = run_gpu(gpu_lib, m, system, pos[k].copy(), types[k].copy(), w, m.r_cut)
    assert len(col) == gold["edges"]
    atoms = np.asarray(gold["forces"]["0"]["atoms"])
    Fo = np.asarray(gold["forces"]["0"]["F"])
    rms = np.sqrt(np.mean(Fo ** 2))
    ferr = np.max(np.abs(F[inv[atoms]] - Fo)) / rms
    eerr = abs(E[0] - gold["energy"]["0"]["E"]) / abs(gold["energy"]["0"]["E"])
    print(f"bulk64k in cell order: E err {eerr:.2e}, F max/rms {ferr:.2e}")
    assert eerr <= E_TOL_F32 and ferr <= F_TOL_F32


def test_largest_admitted_system(gpu_lib):
    """The largest batch the library admits (at most 2^22 atoms): 15,592
    replicas of the 269-bead chain model, 4,194,248 atoms and about 68M
    directed edges, where the per-atom feature arrays span 2^31 - 2^15 bytes
    and the masked-gather offset sits just past their end. Replicas are
    independent, so sampled replicas are checked exactly against the oracle
    on that replica alone (the batch repeats the first 1024 conformations),
    with the fp32 filter at the fp32 bars and the bf16 filter at its own."""
    import dataclasses
    cfg, pos0, types0, w = make_config("md1024")
    N = cfg.system.atoms_per_replica
    R = (1 << 22) // N
    assert R * N <= (1 << 22) < (R + 1) * N
    reps = np.arange(R) % 1024
    pos = pos0.reshape(1024, N, 3)[reps].reshape(-1, 3)
    types = types0.reshape(1024, N)[reps].reshape(-1)
    system = lib_system(gpu_lib, cfg.system, R)
    for dtype in (0, 1):
        m = dataclasses.replace(cfg.model, filter_dtype=dtype)
        E, F, _, col = run_gpu(gpu_lib, m, system, pos, types, w, m.r_cut)
        for r in (0, 7777, R - 1):
            sl = slice(r * N, (r + 1) * N)
            rp, cl = oracle.neighbor_list(pos[sl], 1, N, False, 0.0, m.r_cut)
            Eo, Fo, eps = oracle.energy_forces(oracle_desc(m), w, pos[sl], types[sl], rp, cl,
                                               n_replicas=1, return_eps=True)
            re, rf = assert_energy_forces(E[r:r + 1], F[sl], Eo, Fo, bf16=dtype == 1,
                                          what=f"max size r{r} dtype {dtype}",
                                          eps_abs_sum=[np.abs(eps).sum()])
            print(f"largest batch, dtype {dtype}, replica {r}: {len(col)} edges in all, "
                  f"E rel {re:.2e}, F max/rms {rf:.2e}")
