"""Shared plumbing for the GPU parity tests (inputs, oracle calls, tolerances)."""
from __future__ import annotations

import numpy as np

import oracle
from gen.configs import CONFIGS, make_config

# Parity bars: energy within 1e-5 relative; forces within 1e-4 (max abs) of the
# oracle's force RMS, for fp32 filters. bf16 filters: the oracle uses the same
# bf16-rounded weights but exact activations, so the bars widen to 1e-3 on the
# energy and 5e-2 (max) / 1e-2 (RMS) on the forces.
E_TOL_F32, F_TOL_F32 = 1e-5, 1e-4
E_TOL_BF16, F_TOL_BF16, F_RMS_TOL_BF16 = 1e-3, 5e-2, 1e-2
# fp16 operands in every MLP (W16A16): every activation entering a product is
# rounded to 11 significant bits, so a replica's energy error grows with the
# per-atom energies it sums, not with their (possibly cancelling) total: the
# 16-bit energy bar (1e-3, about two fp16 unit roundoffs) is taken relative to
# sum_i |eps_i|; the force bars are the bf16 ones.
E_TOL_W16_ABS_SUM = 1e-3


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


def assert_energy_forces(E_gpu, F_gpu, E_ref, F_ref, bf16=False, what="", eps_abs_sum=None):
    """bf16: the 16-bit bars; with eps_abs_sum (per replica sum of |eps_i|
    from the oracle) the energy bar is the W16A16 one."""
    E_gpu = np.asarray(E_gpu, dtype=np.float64)
    F_gpu = np.asarray(F_gpu, dtype=np.float64).reshape(-1, 3)
    rel = np.abs(E_gpu - E_ref) / np.maximum(np.abs(E_ref), 1e-30)
    if eps_abs_sum is not None:
        bound = E_TOL_W16_ABS_SUM * np.asarray(eps_abs_sum, dtype=np.float64)
        err = np.abs(E_gpu - E_ref)
        assert np.all(err <= bound), \
            f"{what} energy err {np.max(err / bound) * E_TOL_W16_ABS_SUM:.3e} of sum|eps|"
    else:
        e_tol = E_TOL_BF16 if bf16 else E_TOL_F32
        assert np.all(rel <= e_tol), f"{what} energy rel err {rel.max():.3e} > {e_tol}"
    rms = np.sqrt(np.mean(F_ref ** 2))
    err = np.abs(F_gpu - F_ref)
    if rms == 0.0:            # no forces at all (isolated atoms): demand exact zeros
        assert err.max() == 0.0, f"{what} forces should vanish"
        return rel.max(), 0.0
    f_tol = F_TOL_BF16 if bf16 else F_TOL_F32
    assert err.max() <= f_tol * rms, f"{what} force max err {err.max() / rms:.3e} x rms > {f_tol}"
    if bf16:
        assert np.sqrt(np.mean(err ** 2)) <= F_RMS_TOL_BF16 * rms
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
