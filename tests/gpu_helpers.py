"""Shared plumbing for the GPU parity tests (inputs, oracle calls, tolerances)."""
from __future__ import annotations

import numpy as np

import oracle
from gen.configs import CONFIGS, make_config

# Parity bars: energy within 1e-5 relative; forces within 1e-4 (max abs) of the
# oracle's force RMS, for fp32 filters. bf16 filters: the oracle uses the same
# bf16-rounded weights but exact activations, while the path rounds four
# filter activations per edge to 8 significant bits, so the bars are the
# 16-bit ones that rounding allows: a replica's energy within 1e-3 of
# sum_i |eps_i| (each atom's rounding error does not cancel when the energies
# do), forces within 5e-2 max and 5e-3 RMS of the force RMS. The same
# rounding applied to the oracle's arithmetic, at nine scales across a
# binade, reaches 4.4e-4, 2.9e-2 and 2.9e-3 on one- and five-block models
# (test_16bit_bars); the path itself measured 2.3e-4, 2.3e-2 and 2.7e-3 there. The path's own
# rounding is checked far more tightly against tests.rounding_model
# (test_gpu_rounding_model).
E_TOL_F32, F_TOL_F32 = 1e-5, 1e-4
E_TOL_BF16_ABS_SUM, F_TOL_BF16, F_RMS_TOL_BF16 = 1e-3, 5e-2, 5e-3
# fp16 operands in every MLP (W16A16): every activation entering a product is
# rounded to 11 significant bits, so a replica's energy error grows with the
# per-atom energies it sums, not with their (possibly cancelling) total: the
# energy bar is taken relative to sum_i |eps_i|. Bars at about twice the
# largest measured errors (1.6e-4 of sum |eps_i|, forces 3.6e-3 max and
# 4.9e-4 RMS of the force RMS); the same rounding applied to the oracle's
# arithmetic at nine scales reaches 9.0e-5, 5.2e-3 and 5.7e-4 on one- and
# five-block chain models (test_16bit_bars).
E_TOL_W16_ABS_SUM = 3.5e-4
F_TOL_W16, F_RMS_TOL_W16 = 7e-3, 1e-3


def depth_scale(T):
    """The 16-bit bars above hold for models of up to five interaction blocks;
    every block adds the errors of its own rounded filter and update, which at
    most add up, so deeper models scale them by T / 5 (test_16bit_bars checks
    eight blocks against the scaled bars)."""
    return max(1.0, T / 5.0)


def oracle_desc(m):
    return oracle.ModelDesc(m.n_types, m.D, m.Dr, m.T, m.rbf_min, m.rbf_max, m.r_cut, m.H,
                            m.filter_dtype)


def lib_desc(lib, m):
    return lib.make_desc(m.n_types, m.D, m.Dr, m.T, m.H, m.rbf_min, m.rbf_max, m.r_cut,
                         m.filter_dtype)


def lib_system(lib, s, n_replicas=None):
    R = s.n_replicas if n_replicas is None else n_replicas
    return lib.make_system(R, s.atoms_per_replica, s.periodic, s.box)


def gpu_neighbors(lib, system, pos_np, r_list, capacity=None, ws=None):
    import torch
    n = system.n_replicas * system.atoms_per_replica
    if ws is None:
        ws = lib.Workspace(lib.sn_workspace_size(None, system))
    p = torch.from_numpy(np.ascontiguousarray(pos_np, dtype=np.float32)).cuda().reshape(-1)
    rowptr = torch.full((n + 1,), -7, dtype=torch.int32, device="cuda")
    cap = capacity if capacity is not None else max(1, n * 200)
    col = torch.full((max(cap, 1),), -7, dtype=torch.int32, device="cuda")
    ne = lib.sn_build_neighbors(system, p, r_list, rowptr, col, cap, ws)
    return p, rowptr, col, ne, ws


def oracle_list(system, pos_np, r_list, rp_gpu, col_gpu, what=""):
    """The oracle's own list for the same positions and radius, after checking
    that the GPU's list equals it entry for entry (the oracle is then
    evaluated on a list the GPU did not build)."""
    rp, col = oracle.neighbor_list(np.ascontiguousarray(pos_np, dtype=np.float32),
                                   system.n_replicas, system.atoms_per_replica,
                                   bool(system.periodic), system.box, r_list)
    assert np.array_equal(np.asarray(rp_gpu), rp), f"{what}: GPU rowptr differs from the oracle's"
    assert np.array_equal(np.asarray(col_gpu), col), f"{what}: GPU col differs from the oracle's"
    return rp, col


def assert_energy_forces(E_gpu, F_gpu, E_ref, F_ref, bf16=False, what="", eps_abs_sum=None,
                         w16=False, depth=1.0):
    """bf16: the 16-bit bars (w16: the tighter W16A16 ones) times `depth`
    (depth_scale of the model's block count); their energy bar needs
    eps_abs_sum, the oracle's per-replica sum of |eps_i|."""
    E_gpu = np.asarray(E_gpu, dtype=np.float64)
    F_gpu = np.asarray(F_gpu, dtype=np.float64).reshape(-1, 3)
    rel = np.abs(E_gpu - E_ref) / np.maximum(np.abs(E_ref), 1e-30)
    if bf16:
        assert eps_abs_sum is not None, "16-bit energy bars are taken against sum |eps_i|"
        e_tol = depth * (E_TOL_W16_ABS_SUM if w16 else E_TOL_BF16_ABS_SUM)
        err = np.abs(E_gpu - E_ref) / np.asarray(eps_abs_sum, dtype=np.float64)
        assert np.all(err <= e_tol), f"{what} energy err {err.max():.3e} of sum|eps| > {e_tol}"
    else:
        assert np.all(rel <= E_TOL_F32), f"{what} energy rel err {rel.max():.3e} > {E_TOL_F32}"
    rms = np.sqrt(np.mean(F_ref ** 2))
    err = np.abs(F_gpu - F_ref)
    if rms == 0.0:            # no forces at all (isolated atoms): demand exact zeros
        assert err.max() == 0.0, f"{what} forces should vanish"
        return rel.max(), 0.0
    f_tol = depth * (F_TOL_W16 if w16 else F_TOL_BF16) if bf16 else F_TOL_F32
    assert err.max() <= f_tol * rms, f"{what} force max err {err.max() / rms:.3e} x rms > {f_tol}"
    if bf16:
        e_rms = np.sqrt(np.mean(err ** 2)) / rms
        print(f"{what}: F err rms/rms {e_rms:.2e}")
        assert e_rms <= depth * (F_RMS_TOL_W16 if w16 else F_RMS_TOL_BF16)
    return rel.max(), err.max() / rms


def cutout_forces(cfg, pos, types, w, m, centre, radius, inner):
    """Oracle forces of the atoms within `inner` of atom `centre` of a periodic
    box, from a non-periodic cutout of every atom within `radius` of it.

    An atom's energy depends on positions within T r_c of it, so the force on
    atom i involves positions within 2 T r_c of i: with radius >= inner +
    2 T r_c the cutout gives those forces exactly. Positions are unwrapped
    about the centre by whole box lengths in fp64 (exact), and the cutout's
    list is the oracle's periodic list restricted to pairs inside it (the
    same pairs, since every such pair's minimum image is its unwrapped
    difference)."""
    L = float(np.float32(cfg.system.box))
    p = pos.astype(np.float64)
    u = p - p[centre]
    shift = L * np.round(u / L)
    r = np.linalg.norm(u - shift, axis=1)
    sel = np.nonzero(r < radius)[0]
    idx = -np.ones(len(pos), np.int64)
    idx[sel] = np.arange(len(sel))
    rp, col = oracle.neighbor_list(pos, 1, len(pos), True, cfg.system.box, m.r_cut)
    rows, cols = [0], []
    for a in sel:
        nb = idx[col[rp[a]:rp[a + 1]]]
        nb = np.sort(nb[nb >= 0])
        cols.append(nb)
        rows.append(rows[-1] + len(nb))
    sub_rp = np.asarray(rows, np.int64)
    sub_col = np.concatenate(cols)
    _, Fo = oracle.energy_forces(oracle_desc(m), w, p[sel] - shift[sel], types[sel], sub_rp,
                                 sub_col, n_replicas=1)
    keep = r[sel] < inner
    return sel[keep], Fo[keep]


def open_system(shape, seed=5):
    """One open (non-periodic) system of at least 8192 atoms, the size from
    which the library builds its list from cells over the bounding box. The
    density of the bulk workloads (0.0612 per A^3) unless the shape says
    otherwise; returns float32 positions and the list radius."""
    rng = np.random.default_rng([seed, 7])
    rho, r = 0.0612, 5.0
    if shape == "cube":
        n = 20000
        pos = rng.uniform(0.0, (n / rho) ** (1 / 3), (n, 3))
    elif shape == "ball":           # centred off the origin, negative coordinates too
        n = 16384
        v = rng.normal(size=(n, 3))
        v /= np.linalg.norm(v, axis=1, keepdims=True)
        R = (3 * n / (4 * np.pi * rho)) ** (1 / 3)
        pos = v * R * rng.uniform(0.0, 1.0, (n, 1)) ** (1 / 3) - 7.3
    elif shape == "slab":           # zero thickness: one cell across it
        n = 10000
        pos = np.full((n, 3), 3.25)
        pos[:, :2] = rng.uniform(-200.0, 200.0, (n, 2))
    elif shape == "outlier":        # one far atom: the cell count capped, cells >> r
        n = 9001
        pos = rng.uniform(0.0, ((n - 1) / rho) ** (1 / 3), (n, 3))
        pos[-1] = (1.0e4, -1.0e4, 5.0e3)
    elif shape == "lattice":        # spacings within an ulp or two of the radius, and at it
        inside = float(np.nextafter(np.float32(r), np.float32(0)))
        i, j, k = np.meshgrid(np.arange(32), np.arange(16), np.arange(16), indexing="ij")
        pos = np.stack([i * np.float32(inside), j * np.float32(r), k * np.float32(1.5 * r)],
                       axis=-1).reshape(-1, 3)
    else:
        raise ValueError(shape)
    return np.ascontiguousarray(pos, dtype=np.float32), r
