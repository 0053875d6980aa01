"""GPU MD path: Philox words, noise, BAOAB trajectory vs the oracle, restore,
rebuild guard."""
import numpy as np
import pytest

import oracle
from gen.configs import CONFIGS, make_config, make_weights
from tests.gpu_helpers import lib_desc, lib_system, oracle_desc

pytestmark = pytest.mark.gpu


def test_philox_words_exact(gpu_lib):
    import torch
    rng = np.random.default_rng(0)
    ctr = rng.integers(0, 2**63, size=(5000, 4), dtype=np.int64).view(np.uint64)
    ctr[:10] = 0
    ctr[10:20, 0] = np.uint64(2**64 - 1)
    key = (0xDEADBEEFCAFEBABE, 12345)
    out = torch.empty(5000 * 4, dtype=torch.int64, device="cuda")
    gpu_lib.sn_philox4x64_10(torch.from_numpy(ctr.view(np.int64).ravel()).cuda(), key[0], key[1],
                             out)
    ref = oracle.philox4x64_10(ctr, key)
    assert np.array_equal(out.cpu().numpy().view(np.uint64).reshape(-1, 4), ref)


def _md_setup(lib, name, R, seed=0, gamma=1.0, skin=1.0, rebuild_every=10, filter_f32=True,
              dtype=None, active=True, T=None):
    import torch
    from dataclasses import replace
    cfg, pos, types, w = make_config(name, seed=seed, n_replicas=R)
    m = cfg.model
    if filter_f32 and m.filter_dtype != 0:
        m = replace(m, filter_dtype=0)
    if dtype is not None:
        m = replace(m, filter_dtype=dtype)
    if T is not None:   # another block count: weights of that shape (no biases, so that
        m = replace(m, T=T)   # the energy stays continuous where edges cross the cutoff)
        w = make_weights(m, seed + 7)
    desc = lib_desc(lib, m)
    system = lib_system(lib, cfg.system, R)
    model = lib.sn_model_create(desc, w)
    ws = lib.Workspace(lib.sn_workspace_size(desc, system))
    p = torch.from_numpy(pos).cuda().reshape(-1)
    t = torch.from_numpy(types).cuda()
    params = lib.make_md_params(2.0, 300.0, gamma, 100.0, skin, rebuild_every, 42)
    state = lib.MdState(p, 400 * len(pos), active=active)
    energy = torch.empty(R, dtype=torch.float32, device="cuda")
    return cfg, m, pos, types, w, desc, system, model, ws, t, params, state, energy


@pytest.mark.parametrize("dtype,T,skin,every", [(0, None, 1.0, 10), (3, None, 1.0, 10),
                                                (0, 1, 1.0, 10), (0, 5, 1.0, 10),
                                                (0, None, 0.0, 1000), (0, None, 1.0, 1)])
def test_short_trajectory_matches_oracle(gpu_lib, dtype, T, skin, every):
    """Ten BAOAB steps of 3 chain replicas with the same Philox stream: the
    GPU (fp32, or the fp32 model on fp16 pairs; the chain model's three
    interaction blocks, or one or five) and the oracle (fp64) trajectories
    agree to fp32 accuracy, and the lists are rebuilt on the same steps:
    every 10, or, with no skin, after every step (any motion trips the
    displacement guard), or on a schedule of every step."""
    lib = gpu_lib
    cfg, m, pos, types, w, desc, system, model, ws, t, params, state, energy = _md_setup(
        lib, "cg269x64", 3, dtype=dtype, T=T, skin=skin, rebuild_every=every)
    try:
        lib.sn_md_init(model, system, t, params, state, energy, ws)
        v0 = state.vel.cpu().double().numpy().reshape(-1, 3)
        F0 = state.forces.cpu().double().numpy().reshape(-1, 3)
        lib.sn_md_step(model, system, t, params, state, 10, energy, ws)
        import torch
        torch.cuda.synchronize()
        st = lib.sn_get_device_status(ws)
        assert st[0] == 0, st
        p_gpu = state.pos.cpu().double().numpy().reshape(-1, 3)
        v_gpu = state.vel.cpu().double().numpy().reshape(-1, 3)
        E_gpu = energy.cpu().double().numpy()
        assert state.step == 10
        n_builds = st[2]
    finally:
        lib.sn_model_destroy(model)

    d = oracle_desc(m)
    W = oracle.unpack_weights(d, w)
    v_init = oracle.init_velocities(42, len(pos), 300.0, 100.0)
    assert np.max(np.abs(v0 - v_init)) < 1e-6 * np.max(np.abs(v_init))
    nl = {}

    def rebuild(p):
        nl["l"] = oracle.neighbor_list(np.asarray(p, np.float32), 3, 269, False, 0.0, m.r_cut + skin)

    def forces(p):
        return oracle.energy_forces(d, None, p, types, *nl["l"], n_replicas=3, weights=W)

    rebuild(pos)
    E0, F0o = forces(pos.astype(np.float64))
    assert np.max(np.abs(F0 - F0o)) < 1e-4 * np.sqrt(np.mean(F0o ** 2))
    p_o, v_o, F_o, E_o, nrb = oracle.baoab_run(forces, rebuild, pos, v_init, F0o, dt_fs=2.0,
                                               temperature_K=300.0, gamma_per_ps=1.0,
                                               mass_amu=100.0, skin=skin, rebuild_every=every,
                                               seed=42, step0=0, n_steps=10)
    assert n_builds == 1 + nrb, (n_builds, nrb)       # the GPU count includes the initial build
    assert nrb == (10 if (skin == 0.0 or every == 1) else 1)
    # displacement over 10 steps is ~ 0.03 A; compare against it
    # fp32 positions of up to ~200 A carry ~1e-5 A rounding per update; the
    # displacement over 10 steps is ~0.03 A
    disp = np.max(np.abs(p_o - pos))
    assert np.max(np.abs(p_gpu - p_o)) < 1e-2 * disp + 2e-4
    assert np.max(np.abs(v_gpu - v_o)) < 1e-3 * np.sqrt(np.mean(v_o ** 2))
    assert np.all(np.abs(E_gpu - E_o) <= 1e-4 * np.abs(E_o) + 1e-4)


def test_periodic_trajectory_matches_oracle(gpu_lib):
    """Ten BAOAB steps of a 389-atom periodic box (the bulk model, fp32, a
    rebuild every 5 steps): positions wrap into [0, L) on both sides and are
    compared by minimum image (a value that rounds to L is 0, as in the
    generator and the kernels)."""
    import torch
    lib = gpu_lib
    cfg = CONFIGS["bulk4k"]
    rng = np.random.default_rng(4)
    n, box = 389, 17.9
    L = float(np.float32(box))
    pos = rng.uniform(0, box, (n, 3)).astype(np.float32)
    pos[pos >= np.float32(box)] = 0
    types = rng.integers(0, 4, n).astype(np.int32)
    m = cfg.model
    w = make_weights(m, 6)
    system = lib.make_system(1, n, True, box)
    desc = lib_desc(lib, m)
    model = lib.sn_model_create(desc, w)
    try:
        ws = lib.Workspace(lib.sn_workspace_size(desc, system))
        p = torch.from_numpy(pos).cuda().reshape(-1)
        t = torch.from_numpy(types).cuda()
        params = lib.make_md_params(2.0, 300.0, 1.0, 100.0, 1.0, 5, 42)
        state = lib.MdState(p, 400 * n, active=True)
        energy = torch.empty(1, dtype=torch.float32, device="cuda")
        lib.sn_md_init(model, system, t, params, state, energy, ws)
        lib.sn_md_step(model, system, t, params, state, 10, energy, ws)
        torch.cuda.synchronize()
        st = lib.sn_get_device_status(ws)
        assert st[0] == 0, st
        p_gpu = state.pos.cpu().double().numpy().reshape(-1, 3)
        v_gpu = state.vel.cpu().double().numpy().reshape(-1, 3)
        E_gpu = energy.cpu().double().numpy()
    finally:
        lib.sn_model_destroy(model)
    assert p_gpu.min() >= 0 and p_gpu.max() < L
    d = oracle_desc(m)
    W = oracle.unpack_weights(d, w)
    v_init = oracle.init_velocities(42, n, 300.0, 100.0)
    nl = {}

    def rebuild(q):
        q32 = np.asarray(q, np.float32)
        q32[q32 >= np.float32(box)] = 0
        nl["l"] = oracle.neighbor_list(q32, 1, n, True, box, m.r_cut + 1.0)

    def forces(q):
        return oracle.energy_forces(d, None, q, types, *nl["l"], n_replicas=1, periodic=True,
                                    box=box, weights=W)

    rebuild(pos)
    E0, F0 = forces(pos.astype(np.float64))
    p_o, v_o, F_o, E_o, nrb = oracle.baoab_run(forces, rebuild, pos, v_init, F0, dt_fs=2.0,
                                               temperature_K=300.0, gamma_per_ps=1.0,
                                               mass_amu=100.0, skin=1.0, rebuild_every=5, seed=42,
                                               step0=0, n_steps=10, periodic=True, box=box)
    assert st[2] == 1 + nrb
    dp = p_gpu - p_o
    dp -= L * np.round(dp / L)
    disp = p_o - pos
    disp -= L * np.round(disp / L)
    assert np.max(np.abs(dp)) < 1e-2 * np.max(np.abs(disp)) + 2e-4
    assert np.max(np.abs(v_gpu - v_o)) < 1e-3 * np.sqrt(np.mean(v_o ** 2))
    assert np.all(np.abs(E_gpu - E_o) <= 1e-4 * np.abs(E_o) + 1e-4)


def test_restore_replays_bitwise(gpu_lib):
    import torch
    lib = gpu_lib
    cfg, m, pos, types, w, desc, system, model, ws, t, params, state, energy = _md_setup(
        lib, "cg269x64", 2, rebuild_every=5)
    try:
        lib.sn_md_init(model, system, t, params, state, energy, ws)
        lib.sn_md_step(model, system, t, params, state, 7, energy, ws)
        snap = {k: getattr(state, k).clone() for k in
                ("pos", "vel", "forces", "pos_at_build", "rowptr", "col")}
        step = state.step
        lib.sn_md_step(model, system, t, params, state, 9, energy, ws)
        a = (state.pos.clone(), state.vel.clone(), energy.clone())
        for k, v in snap.items():
            getattr(state, k).copy_(v)
        state.step = step
        lib.sn_md_step(model, system, t, params, state, 9, energy, ws)
        torch.cuda.synchronize()
        assert torch.equal(a[0], state.pos) and torch.equal(a[1], state.vel)
        assert torch.equal(a[2], energy)
    finally:
        lib.sn_model_destroy(model)


def test_skin_guard_forces_rebuild(gpu_lib):
    """With a tiny skin the displacement guard must rebuild between scheduled
    rebuilds; with a huge cadence only the guard rebuilds."""
    import torch
    lib = gpu_lib
    cfg, m, pos, types, w, desc, system, model, ws, t, params, state, energy = _md_setup(
        lib, "cg269x64", 2, skin=0.02, rebuild_every=1000)
    try:
        lib.sn_md_init(model, system, t, params, state, energy, ws)
        lib.sn_md_step(model, system, t, params, state, 20, energy, ws)
        st, det, nrb = lib.sn_get_device_status(ws)
        assert st == 0
        assert nrb >= 3, f"only {nrb} builds"
        # the list in the state is the exact list of the current positions at r_cut + skin
        # whenever a rebuild just happened; check the forces against a fresh evaluation
        p = state.pos.clone()
        rowptr = torch.zeros_like(state.rowptr)
        col = torch.zeros_like(state.col)
        lib.sn_build_neighbors(system, p, m.r_cut + 0.02, rowptr, col, col.numel(), ws)
        e2 = torch.empty_like(energy)
        f2 = torch.empty_like(state.forces)
        lib.sn_energy_forces(model, system, p, t, rowptr, col, e2, f2, ws)
        torch.cuda.synchronize()
        assert torch.allclose(e2, energy, rtol=1e-6, atol=0)
    finally:
        lib.sn_model_destroy(model)


def test_scheduled_rebuilds_counted_once_each(gpu_lib):
    """With a 3 A skin the guard cannot trip in 20 steps of 2 fs (the beads
    move ~0.1 A), so the builds are exactly the initial one and the scheduled
    ones at steps 4, 9, 14 and 19 (every 5), each counted once, split over
    two calls."""
    lib = gpu_lib
    cfg, m, pos, types, w, desc, system, model, ws, t, params, state, energy = _md_setup(
        lib, "cg269x64", 2, skin=3.0, rebuild_every=5)
    try:
        lib.sn_md_init(model, system, t, params, state, energy, ws)
        lib.sn_md_step(model, system, t, params, state, 7, energy, ws)
        lib.sn_md_step(model, system, t, params, state, 13, energy, ws)
        st, det, nrb = lib.sn_get_device_status(ws)
        assert st == 0
        assert nrb == 1 + 4, f"{nrb} builds"
    finally:
        lib.sn_model_destroy(model)


def test_zero_model_keeps_temperature(gpu_lib):
    """Zero weights give zero forces: the O step is then the exact OU process
    and the kinetic temperature stays at 300 K."""
    import torch
    lib = gpu_lib
    cfg = CONFIGS["cg269x64"]
    m = cfg.model
    R = 64
    from gen.configs import make_system
    pos, types = make_system(cfg.system, m.n_types, 0, R)
    w = np.zeros(lib.sn_model_weight_count(lib_desc(lib, m)), np.float32)
    desc = lib_desc(lib, m)
    system = lib_system(lib, cfg.system, R)
    model = lib.sn_model_create(desc, w)
    try:
        ws = lib.Workspace(lib.sn_workspace_size(desc, system))
        params = lib.make_md_params(2.0, 300.0, 20.0, 100.0, 2.0, 10, 7)
        state = lib.MdState(torch.from_numpy(pos).cuda().reshape(-1), 400 * len(pos))
        energy = torch.empty(R, dtype=torch.float32, device="cuda")
        t = torch.from_numpy(types).cuda()
        lib.sn_md_init(model, system, t, params, state, energy, ws)
        lib.sn_md_step(model, system, t, params, state, 30, energy, ws)
        torch.cuda.synchronize()
        assert torch.all(state.forces == 0)
        v = state.vel.cpu().double().numpy().reshape(-1, 3)
        ke = 0.5 * 100.0 * np.sum(v ** 2, axis=1) / oracle.md.KAPPA
        assert abs(ke.mean() / (1.5 * oracle.md.KB * 300.0) - 1) < 0.03
    finally:
        lib.sn_model_destroy(model)


def test_active_list(gpu_lib):
    """The per-step active list: at initialisation it is exactly the oracle's
    list at r_cut (1 + 2^-10); after 25 steps (with rebuilds and without) it
    holds every pair inside r_cut and none beyond the keep radius, each row
    in the skin list's order; and trajectories with and without it agree to
    rounding (listed pairs beyond r_cut contribute nothing)."""
    import torch
    lib = gpu_lib
    R = 4
    cfg, m, pos, types, w, desc, system, model, ws, t, params, state, energy = _md_setup(
        lib, "md1024", R, filter_f32=False, rebuild_every=10)
    N = cfg.system.atoms_per_replica
    r_keep = float(np.float32(m.r_cut + m.r_cut / 1024.0))
    try:
        lib.sn_md_init(model, system, t, params, state, energy, ws)
        torch.cuda.synchronize()
        rp_a = state.rowptr_active.cpu().numpy()
        col_a = state.col_active[:rp_a[-1]].cpu().numpy()
        rp_o, col_o = oracle.neighbor_list(state.pos.cpu().numpy().reshape(-1, 3), R, N, False,
                                           0.0, r_keep)
        assert np.array_equal(rp_a, rp_o) and np.array_equal(col_a, col_o)
        lib.sn_md_step(model, system, t, params, state, 25, energy, ws)
        torch.cuda.synchronize()
        assert lib.sn_get_device_status(ws)[0] == 0
        p_now = state.pos.cpu().numpy().reshape(-1, 3)
        rp_a = state.rowptr_active.cpu().numpy()
        col_a = state.col_active[:rp_a[-1]].cpu().numpy()
        rp_s = state.rowptr.cpu().numpy()
        col_s = state.col[:rp_s[-1]].cpu().numpy()
        rp_c, col_c = oracle.neighbor_list(p_now, R, N, False, 0.0, m.r_cut)
        rp_k, col_k = oracle.neighbor_list(p_now, R, N, False, 0.0, r_keep)
        for i in range(R * N):
            a = col_a[rp_a[i]:rp_a[i + 1]]
            assert set(col_c[rp_c[i]:rp_c[i + 1]]) <= set(a) <= set(col_k[rp_k[i]:rp_k[i + 1]])
            s = list(col_s[rp_s[i]:rp_s[i + 1]])
            assert [s.index(j) for j in a] == sorted(s.index(j) for j in a)
        E_act = energy.cpu().double().numpy()
        P_act = p_now.astype(np.float64)
    finally:
        lib.sn_model_destroy(model)
    cfg, m, pos, types, w, desc, system, model, ws, t, params, state, energy = _md_setup(
        lib, "md1024", R, filter_f32=False, rebuild_every=10, active=False)
    try:
        lib.sn_md_init(model, system, t, params, state, energy, ws)
        lib.sn_md_step(model, system, t, params, state, 25, energy, ws)
        torch.cuda.synchronize()
        E_full = energy.cpu().double().numpy()
        P_full = state.pos.cpu().double().numpy().reshape(-1, 3)
    finally:
        lib.sn_model_destroy(model)
    disp = np.max(np.abs(P_full - pos))
    assert np.max(np.abs(P_act - P_full)) < 1e-3 * disp
    assert np.all(np.abs(E_act - E_full) <= 1e-4 * np.abs(E_full))


def test_nonfinite_position_is_reported(gpu_lib):
    """A NaN written into one bead's position: the next step's B-A-O-A sees
    it and the device status becomes SN_ERR_NONFINITE with detail -(1 + atom)
    (before, the bead silently lost its edges and the status stayed SN_OK).
    An infinite velocity of another bead is reported the same way."""
    import torch
    lib = gpu_lib
    cfg, m, pos, types, w, desc, system, model, ws, t, params, state, energy = _md_setup(
        lib, "cg269x64", 2)
    try:
        lib.sn_md_init(model, system, t, params, state, energy, ws)
        assert lib.sn_get_device_status(ws)[0] == 0
        state.pos[3 * 300 + 1] = float("nan")
        lib.sn_md_step(model, system, t, params, state, 1, energy, ws)
        st, det, _ = lib.sn_get_device_status(ws)
        assert st == lib.SN_ERR_NONFINITE and det == -(1 + 300), (st, det)
    finally:
        lib.sn_model_destroy(model)
    cfg, m, pos, types, w, desc, system, model, ws, t, params, state, energy = _md_setup(
        lib, "cg269x64", 2)
    try:
        lib.sn_md_init(model, system, t, params, state, energy, ws)
        state.vel[3 * 17 + 2] = float("inf")
        lib.sn_md_step(model, system, t, params, state, 1, energy, ws)
        st, det, _ = lib.sn_get_device_status(ws)
        assert st == lib.SN_ERR_NONFINITE and det == -(1 + 17), (st, det)
    finally:
        lib.sn_model_destroy(model)


@pytest.mark.parametrize("periodic", [False, True])
def test_nonfinite_position_in_neighbour_build(gpu_lib, periodic):
    """sn_build_neighbors on positions with one NaN coordinate (all-pairs
    search, and the cell list of a periodic cube) reports the atom."""
    import torch
    lib = gpu_lib
    rng = np.random.default_rng(5)
    if periodic:
        n, box = 4000, 40.0
        pos = rng.uniform(0, box, (n, 3)).astype(np.float32)
        system = lib.make_system(1, n, True, box)
    else:
        n, box = 300, 0.0
        pos = rng.uniform(0, 30.0, (n, 3)).astype(np.float32)
        system = lib.make_system(1, n, False, 0.0)
    pos[123, 0] = np.nan
    ws = lib.Workspace(lib.sn_workspace_size(None, system))
    p = torch.from_numpy(pos).cuda().reshape(-1)
    rowptr = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    col = torch.zeros(n * 200, dtype=torch.int32, device="cuda")
    lib.sn_build_neighbors(system, p, 5.0, rowptr, col, n * 200, ws)
    st, det, _ = lib.sn_get_device_status(ws)
    assert st == lib.SN_ERR_NONFINITE and det == -(1 + 123), (st, det)


@pytest.mark.parametrize("dtype", [1, 2])
def test_short_trajectory_16bit_active_list(gpu_lib, dtype):
    """The MD workload's own precision and path (a bf16 filter, the update
    and readout layers on fp16 pairs; or W16A16), the per-step active list,
    ten BAOAB steps of 3 replicas against the oracle with the same rounded
    weights and exact activations. Bars follow from the 16-bit force bar:
    a force error of at most F_TOL F_rms per step moves velocities by at
    most that times dt kappa / m per step, and positions by dt times that."""
    import torch
    from tests.gpu_helpers import E_TOL_BF16_ABS_SUM, E_TOL_W16_ABS_SUM, F_TOL_BF16, F_TOL_W16
    E_TOL, F_TOL = (E_TOL_BF16_ABS_SUM, F_TOL_BF16) if dtype == 1 else (E_TOL_W16_ABS_SUM,
                                                                        F_TOL_W16)
    lib = gpu_lib
    nsteps = 10
    cfg, m, pos, types, w, desc, system, model, ws, t, params, state, energy = _md_setup(
        lib, "md1024", 3, filter_f32=False, dtype=dtype, active=True)
    assert m.filter_dtype == dtype
    try:
        lib.sn_md_init(model, system, t, params, state, energy, ws)
        F0 = state.forces.cpu().double().numpy().reshape(-1, 3)
        lib.sn_md_step(model, system, t, params, state, nsteps, energy, ws)
        torch.cuda.synchronize()
        st = lib.sn_get_device_status(ws)
        assert st[0] == 0, st
        p_gpu = state.pos.cpu().double().numpy().reshape(-1, 3)
        v_gpu = state.vel.cpu().double().numpy().reshape(-1, 3)
        E_gpu = energy.cpu().double().numpy()
    finally:
        lib.sn_model_destroy(model)
    d = oracle_desc(m)
    W = oracle.unpack_weights(d, w)
    v_init = oracle.init_velocities(42, len(pos), 300.0, 100.0)
    nl = {}

    def rebuild(p):
        nl["l"] = oracle.neighbor_list(np.asarray(p, np.float32), 3, 269, False, 0.0, m.r_cut + 1.0)

    def forces(p):
        return oracle.energy_forces(d, None, p, types, *nl["l"], n_replicas=3, weights=W)

    rebuild(pos)
    E0, F0o = forces(pos.astype(np.float64))
    f_rms = np.sqrt(np.mean(F0o ** 2))
    assert np.max(np.abs(F0 - F0o)) <= F_TOL * f_rms
    p_o, v_o, F_o, E_o, _ = oracle.baoab_run(forces, rebuild, pos, v_init, F0o, dt_fs=2.0,
                                             temperature_K=300.0, gamma_per_ps=1.0,
                                             mass_amu=100.0, skin=1.0, rebuild_every=10, seed=42,
                                             step0=0, n_steps=nsteps)
    kick = 2.0 * oracle.md.KAPPA / 100.0                 # dt kappa / m per step
    dv_bar = nsteps * kick * F_TOL * f_rms + 1e-3 * np.sqrt(np.mean(v_o ** 2))
    disp = np.max(np.abs(p_o - pos))
    dp_bar = nsteps * 2.0 * dv_bar + 1e-2 * disp + 2e-4
    dv = np.max(np.abs(v_gpu - v_o))
    dp = np.max(np.abs(p_gpu - p_o))
    _, _, eps = oracle.energy_forces(d, None, p_o, types, *nl["l"], n_replicas=3, weights=W,
                                     return_eps=True)
    de = np.max(np.abs(E_gpu - E_o) / np.abs(eps).reshape(3, -1).sum(axis=1))
    print(f"dtype {dtype} trajectory: dv {dv:.2e} (bar {dv_bar:.2e}), dp {dp:.2e} (bar {dp_bar:.2e}), "
          f"E err {de:.2e} of sum|eps|")
    assert dv <= dv_bar and dp <= dp_bar
    assert de <= E_TOL
