"""Pins for the oracle's energy and forces.

Each check ties the oracle to something other than itself: a scalar closed
form, central finite differences, torch.autograd on an independently written
forward, exact symmetries of a distance-only energy, and special cases that
reduce to simpler computations."""
import math

import numpy as np
import pytest
import torch

from gen.configs import CONFIGS, make_config, make_weights
from gen.systems import model_weights
from oracle.neighbors import neighbor_list
from oracle.schnet import ModelDesc, energy, energy_forces, forward_trace, unpack_weights


def desc_of(cfg):
    m = cfg.model
    return ModelDesc(m.n_types, m.D, m.Dr, m.T, m.rbf_min, m.rbf_max, m.r_cut, m.H, m.filter_dtype)


def small_chain(n=24, seed=3, bias=0.0):
    """A cg32-like chain model shrunk for speed, with optional biases."""
    rng = np.random.default_rng(seed)
    steps = rng.standard_normal((n - 1, 3))
    steps = 3.8 * steps / np.linalg.norm(steps, axis=1, keepdims=True)
    pos = np.vstack([np.zeros(3), np.cumsum(steps, 0)]).astype(np.float32)
    pos += rng.normal(0, 0.2, pos.shape).astype(np.float32)
    desc = ModelDesc(n_types=3, D=16, Dr=12, T=2, rbf_min=0.0, rbf_max=10.0, r_cut=10.0, H=8)
    w = model_weights(np.random.default_rng([seed, 2]), 3, 16, 12, 2, 8, bias_scale=bias)
    types = rng.integers(0, 3, n).astype(np.int32)
    return desc, w, pos, types


# ---------------------------------------------------------------- closed forms
def _ssp(x):
    return math.log1p(math.exp(x)) - math.log(2.0)


def _sig(x):
    return 1.0 / (1.0 + math.exp(-x))


def test_two_atom_scalar_closed_form():
    """D = 1, Dr = 2, T = 1, H = 1: the energy of two like atoms at distance d
    and its derivative, written out by hand in scalar arithmetic."""
    rc = 5.0
    desc = ModelDesc(n_types=1, D=1, Dr=2, T=1, rbf_min=0.0, rbf_max=rc, r_cut=rc, H=1)
    e, p, q, c1, r0, c2, a0, b0, a1, b1, o1, k1, o2, k2 = (
        0.7, 0.9, -1.3, 0.1, 1.7, -0.2, 0.8, 0.05, -1.1, 0.3, 1.4, -0.1, 0.6, 0.25)
    flat = np.array([e, p, q, c1, r0, c2, a0, b0, a1, b1, o1, k1, o2, k2], dtype=np.float32)
    flat64 = flat.astype(np.float64)
    e, p, q, c1, r0, c2, a0, b0, a1, b1, o1, k1, o2, k2 = flat64
    pos = np.array([[0.3, -0.2, 0.1], [2.1, 1.4, -0.9]], dtype=np.float32)
    rowptr = np.array([0, 1, 2])
    col = np.array([1, 0])
    u = pos[0].astype(np.float64) - pos[1].astype(np.float64)
    d = math.sqrt(float(u @ u))
    sig = rc                                   # spacing of two centres on [0, rc]
    g0 = math.exp(-d * d / (2 * sig * sig))
    g1 = math.exp(-(d - rc) ** 2 / (2 * sig * sig))
    C = 0.5 * (math.cos(math.pi * d / rc) + 1)
    a = (p * g0 + q * g1) * C + c1
    w = _ssp(a) * r0 + c2
    h = e * w
    xp = e + _ssp(h * a0 + b0) * a1 + b1
    eps = _ssp(xp * o1 + k1) * o2 + k2
    E_ref = 2 * eps
    dg0 = -d / (sig * sig) * g0
    dg1 = -(d - rc) / (sig * sig) * g1
    dC = -0.5 * math.pi / rc * math.sin(math.pi * d / rc)
    dbt = (p * dg0 + q * dg1) * C + (p * g0 + q * g1) * dC
    dE_dd = 2 * o2 * _sig(xp * o1 + k1) * o1 * _sig(h * a0 + b0) * a1 * a0 * e * r0 * _sig(a) * dbt
    E, F = energy_forces(desc, flat, pos, np.zeros(2, np.int32), rowptr, col)
    assert abs(E[0] - E_ref) < 1e-13
    F0_ref = -dE_dd * u / d
    assert np.max(np.abs(F[0] - F0_ref)) < 1e-13
    assert np.max(np.abs(F[1] + F0_ref)) < 1e-13


def test_T0_is_readout_of_embedding():
    desc, w, pos, types = small_chain()
    d0 = ModelDesc(desc.n_types, desc.D, desc.Dr, 0, desc.rbf_min, desc.rbf_max, desc.r_cut, desc.H)
    W = unpack_weights(desc, w)
    # T = 0 vector: embedding then readout parameters only
    nb = desc.Dr * desc.D + desc.D + 3 * (desc.D * desc.D + desc.D)
    flat0 = np.concatenate([w[:desc.n_types * desc.D], w[desc.n_types * desc.D + desc.T * nb:]])
    rp, col = neighbor_list(pos, 1, len(pos), False, 0.0, desc.r_cut)
    E, F = energy_forces(d0, flat0, pos, types, rp, col)
    x = W["emb"][types]
    z = x @ W["Wo1"] + W["co1"]
    eps = (np.logaddexp(0, z) - np.log(2)) @ W["Wo2"] + W["co2"][0]
    assert abs(E[0] - eps.sum()) < 1e-12
    assert np.all(F == 0)


def test_edges_beyond_cutoff_give_isolated_atoms():
    """A list built with a radius larger than every pair distance but a model
    whose cutoff is below every pair distance: every edge is masked and, with
    zero biases, each atom keeps its embedding through the blocks."""
    desc, w, pos, types = small_chain()
    far = ModelDesc(desc.n_types, desc.D, desc.Dr, desc.T, 0.0, 1.0, 1.0, desc.H)
    rp, col = neighbor_list(pos, 1, len(pos), False, 0.0, 200.0)
    assert len(col) == len(pos) * (len(pos) - 1)
    E, F = energy_forces(far, w, pos, types, rp, col)
    W = unpack_weights(far, w)
    z = W["emb"][types] @ W["Wo1"]
    eps = (np.logaddexp(0, z) - np.log(2)) @ W["Wo2"]
    assert abs(E[0] - eps.sum()) < 1e-12
    assert np.all(F == 0)


def test_zero_filter_output_gives_zero_messages():
    desc, w, pos, types = small_chain(bias=0.3)
    W = unpack_weights(desc, w)
    off = desc.n_types * desc.D
    w2 = w.copy()
    for t in range(desc.T):
        base = off + t * (desc.Dr * desc.D + desc.D + 3 * (desc.D * desc.D + desc.D))
        s = base + desc.Dr * desc.D + desc.D            # start of Wf2
        w2[s:s + desc.D * desc.D + desc.D] = 0.0        # Wf2 and cf2
    rp, col = neighbor_list(pos, 1, len(pos), False, 0.0, desc.r_cut)
    eps, tape = forward_trace(desc, w2, pos, types, rp, col)
    for (x, a1, wf, h, au) in tape:
        assert np.all(h == 0)
    # x only moves by the constant update ssp(cu1) Wu2 + cu2
    x = W["emb"][types]
    for blk in W["blocks"]:
        x = x + (np.logaddexp(0, blk["cu1"]) - np.log(2)) @ blk["Wu2"] + blk["cu2"]
    z = x @ W["Wo1"] + W["co1"]
    ref = (np.logaddexp(0, z) - np.log(2)) @ W["Wo2"] + W["co2"][0]
    assert np.max(np.abs(eps - ref)) < 1e-12


def test_aggregation_equals_dense_adjacency_product():
    desc, w, pos, types = small_chain(n=12)
    rp, col = neighbor_list(pos, 1, len(pos), False, 0.0, desc.r_cut)
    eps, tape = forward_trace(desc, w, pos, types, rp, col)
    n = len(pos)
    dst = np.repeat(np.arange(n), np.diff(rp))
    for (x, a1, wf, h, au) in tape:
        Wd = np.zeros((n, n, desc.D))
        Wd[dst, col] = wf                       # dense filter tensor, zero off-graph
        h_dense = np.einsum("ijd,jd->id", Wd, x)
        assert np.max(np.abs(h - h_dense)) < 1e-12


# ---------------------------------------------------------------- derivatives
def test_forces_match_central_differences():
    desc, w, pos, types = small_chain(n=20)
    rp, col = neighbor_list(pos, 1, len(pos), False, 0.0, desc.r_cut + 1.0)   # skin list
    W = unpack_weights(desc, w)
    E0, F = energy_forces(desc, None, pos, types, rp, col, weights=W)
    p64 = pos.astype(np.float64)
    h = 1e-5
    num = np.zeros_like(p64)
    for i in range(len(p64)):
        for ax in range(3):
            pp, pm = p64.copy(), p64.copy()
            pp[i, ax] += h
            pm[i, ax] -= h
            num[i, ax] = -(energy(desc, None, pp, types, rp, col, weights=W)[0]
                           - energy(desc, None, pm, types, rp, col, weights=W)[0]) / (2 * h)
    scale = np.sqrt(np.mean(F ** 2))
    assert np.max(np.abs(num - F)) < 1e-7 * max(scale, 1.0)


def test_coincident_atoms_match_central_differences():
    """Two atoms at one position: E depends on their pair only through
    d = |u|, which is even in u, so a central difference along any coordinate
    of either atom cancels that pair's kink exactly. The oracle's convention
    for the pair's force term (zero where d = 0, as u = 0) must reproduce it."""
    desc, w, pos, types = small_chain(n=12)
    pos = pos.copy()
    pos[4] = pos[7]
    rp, col = neighbor_list(pos, 1, len(pos), False, 0.0, desc.r_cut)
    assert 7 in col[rp[4]:rp[5]] and 4 in col[rp[7]:rp[8]]
    W = unpack_weights(desc, w)
    E0, F = energy_forces(desc, None, pos, types, rp, col, weights=W)
    assert np.all(np.isfinite(E0)) and np.all(np.isfinite(F))
    p64 = pos.astype(np.float64)
    h = 1e-5
    scale = np.sqrt(np.mean(F ** 2))
    for i in (4, 7, 5):
        for ax in range(3):
            pp, pm = p64.copy(), p64.copy()
            pp[i, ax] += h
            pm[i, ax] -= h
            num = -(energy(desc, None, pp, types, rp, col, weights=W)[0]
                    - energy(desc, None, pm, types, rp, col, weights=W)[0]) / (2 * h)
            assert abs(num - F[i, ax]) < 1e-7 * max(scale, 1.0), (i, ax, num, F[i, ax])


def _torch_energy(desc, W, pos, types, rowptr, col, periodic=False, box=0.0):
    """Second implementation of the forward in torch (fp64, CPU), aggregation by
    index_add_; differentiated by torch.autograd."""
    t = lambda a: torch.as_tensor(a, dtype=torch.float64)
    src = torch.as_tensor(np.asarray(col), dtype=torch.long)
    dst = torch.repeat_interleave(torch.arange(len(rowptr) - 1), torch.as_tensor(np.diff(rowptr)))
    r = pos
    u = r[dst] - r[src]
    if periodic:
        L = float(np.float32(box))
        u = u - L * torch.round(u.detach() / L)
    d = torch.linalg.vector_norm(u, dim=1)
    step = (desc.rbf_max - desc.rbf_min) / (desc.Dr - 1)
    mu = desc.rbf_min + step * torch.arange(desc.Dr, dtype=torch.float64)
    g = torch.exp(-((d[:, None] - mu) ** 2) / (2 * step ** 2))
    inside = d < desc.r_cut
    C = torch.where(inside, 0.5 * (torch.cos(math.pi * d / desc.r_cut) + 1), torch.zeros_like(d))
    bt = g * C[:, None]
    sspt = lambda z: torch.logaddexp(z, torch.zeros_like(z)) - math.log(2.0)
    x = t(W["emb"])[torch.as_tensor(types, dtype=torch.long)]
    for blk in W["blocks"]:
        wf = sspt(bt @ t(blk["Wf1"]) + t(blk["cf1"])) @ t(blk["Wf2"]) + t(blk["cf2"])
        wf = wf * inside[:, None]
        hh = torch.zeros_like(x).index_add_(0, dst, x[src] * wf)
        x = x + sspt(hh @ t(blk["Wu1"]) + t(blk["cu1"])) @ t(blk["Wu2"]) + t(blk["cu2"])
    eps = sspt(x @ t(W["Wo1"]) + t(W["co1"])) @ t(W["Wo2"]) + t(W["co2"])[0]
    return eps.sum()


@pytest.mark.parametrize("name", ["cg32", "bulk4k_small"])
def test_forces_match_torch_autograd(name):
    if name == "cg32":
        cfg, pos, types, w = make_config("cg32", bias_scale=0.1)
        desc = desc_of(cfg)
        periodic, box = False, 0.0
    else:
        cfg = CONFIGS["bulk4k"]
        desc = desc_of(cfg)
        rng = np.random.default_rng(9)
        box = 16.0
        pos = rng.uniform(0, box, (256, 3)).astype(np.float32)   # same density as bulk4k
        types = rng.integers(0, 4, 256).astype(np.int32)
        w = make_weights(cfg.model, 1, bias_scale=0.1)
        periodic = True
    rp, col = neighbor_list(pos, 1, len(pos), periodic, box, desc.r_cut)
    W = unpack_weights(desc, w)
    E, F = energy_forces(desc, None, pos, types, rp, col, periodic=periodic, box=box, weights=W)
    pt = torch.tensor(pos.astype(np.float64), requires_grad=True)
    Et = _torch_energy(desc, W, pt, types, rp, col, periodic, box)
    Et.backward()
    assert abs(E[0] - Et.item()) < 1e-10 * max(1.0, abs(E[0]))
    Ft = -pt.grad.numpy()
    assert np.max(np.abs(F - Ft)) < 1e-10 * max(1.0, np.sqrt(np.mean(F ** 2)))


# ---------------------------------------------------------------- invariances
def _rotation(seed):
    q, _ = np.linalg.qr(np.random.default_rng(seed).standard_normal((3, 3)))
    return q * np.sign(np.linalg.det(q))


def test_rotation_translation_permutation_and_net_force():
    cfg, pos, types, w = make_config("cg32")
    desc = desc_of(cfg)
    W = unpack_weights(desc, w)
    p64 = pos.astype(np.float64)
    rp, col = neighbor_list(pos, 1, 32, False, 0.0, desc.r_cut + 2.0)
    E, F = energy_forces(desc, None, p64, types, rp, col, weights=W)
    R = _rotation(1)
    E2, F2 = energy_forces(desc, None, p64 @ R.T + np.array([3.0, -7.0, 11.0]), types, rp, col,
                           weights=W)
    assert abs(E2[0] - E[0]) < 1e-12 * max(1, abs(E[0]))
    assert np.max(np.abs(F2 - F @ R.T)) < 1e-11
    assert np.max(np.abs(F.sum(axis=0))) < 1e-11
    assert np.max(np.abs(np.cross(p64, F).sum(axis=0))) < 1e-10
    perm = np.random.default_rng(2).permutation(32)
    pp = pos[perm]
    rp3, col3 = neighbor_list(pp, 1, 32, False, 0.0, desc.r_cut + 2.0)
    E3, F3 = energy_forces(desc, None, pp, types[perm], rp3, col3, weights=W)
    assert abs(E3[0] - E[0]) < 1e-12 * max(1, abs(E[0]))
    assert np.max(np.abs(F3 - F[perm])) < 1e-11


def test_periodic_translation_and_cube_rotation():
    cfg = CONFIGS["bulk4k"]
    desc = desc_of(cfg)
    rng = np.random.default_rng(4)
    box = 16.0
    pos = rng.uniform(0, box, (256, 3)).astype(np.float32)
    types = rng.integers(0, 4, 256).astype(np.int32)
    W = unpack_weights(desc, make_weights(cfg.model, 0))
    rp, col = neighbor_list(pos, 1, 256, True, box, desc.r_cut)
    E, F = energy_forces(desc, None, pos, types, rp, col, periodic=True, box=box, weights=W)
    # shift by a vector and wrap back into the cube
    sh = np.mod(pos.astype(np.float64) + np.array([5.25, -3.5, 9.75]), box).astype(np.float32)
    sh[sh >= np.float32(box)] = 0
    rp2, col2 = neighbor_list(sh, 1, 256, True, box, desc.r_cut)
    E2, F2 = energy_forces(desc, None, sh, types, rp2, col2, periodic=True, box=box, weights=W)
    assert abs(E2[0] - E[0]) < 1e-5 * abs(E[0])      # fp32 rounding of the shifted inputs
    assert np.max(np.abs(F2 - F)) < 1e-4 * np.sqrt(np.mean(F ** 2))
    # 90 degree rotation about z maps the cube onto itself: (x, y) -> (L - y, x)
    rot = np.stack([np.float32(box) - pos[:, 1], pos[:, 0], pos[:, 2]], axis=1).astype(np.float32)
    rot[rot >= np.float32(box)] = 0
    rp3, col3 = neighbor_list(rot, 1, 256, True, box, desc.r_cut)
    E3, F3 = energy_forces(desc, None, rot, types, rp3, col3, periodic=True, box=box, weights=W)
    assert abs(E3[0] - E[0]) < 1e-5 * abs(E[0])
    Fr = np.stack([-F[:, 1], F[:, 0], F[:, 2]], axis=1)
    assert np.max(np.abs(F3 - Fr)) < 1e-4 * np.sqrt(np.mean(F ** 2))
    assert np.max(np.abs(F.sum(axis=0))) < 1e-10


def test_simple_cubic_lattice_has_zero_force():
    """Single species on a simple cubic lattice, spacing a, cutoff between a and
    a*sqrt(2): every atom has exactly six equivalent neighbours, so every
    per-atom energy is equal and every force vanishes."""
    a, n = 3.0, 5
    L = a * n
    g = np.arange(n) * a + 0.5
    pos = np.stack(np.meshgrid(g, g, g, indexing="ij"), -1).reshape(-1, 3).astype(np.float32)
    desc = ModelDesc(n_types=1, D=16, Dr=10, T=3, rbf_min=0.0, rbf_max=3.5, r_cut=3.5, H=8)
    w = model_weights(np.random.default_rng(7), 1, 16, 10, 3, 8, bias_scale=0.2)
    rp, col = neighbor_list(pos, 1, len(pos), True, L, 3.5)
    assert np.all(np.diff(rp) == 6)
    E, F, eps = energy_forces(desc, w, pos, np.zeros(len(pos), np.int32), rp, col, 1, True, L,
                              return_eps=True)
    assert np.max(np.abs(F)) < 1e-12
    assert np.max(eps) - np.min(eps) < 1e-12


def test_replicas_are_independent():
    cfg, pos, types, w = make_config("cg269x64", n_replicas=3)
    desc = desc_of(cfg)
    W = unpack_weights(desc, w)
    rp, col = neighbor_list(pos, 3, 269, False, 0.0, desc.r_cut)
    E, F = energy_forces(desc, None, pos, types, rp, col, n_replicas=3, weights=W)
    for r in range(3):
        p1 = pos[r * 269:(r + 1) * 269]
        rp1, col1 = neighbor_list(p1, 1, 269, False, 0.0, desc.r_cut)
        E1, F1 = energy_forces(desc, None, p1, types[:269], rp1, col1, weights=W)
        assert abs(E1[0] - E[r]) < 1e-12 * max(1.0, abs(E[r]))
        assert np.max(np.abs(F1 - F[r * 269:(r + 1) * 269])) < 1e-12
