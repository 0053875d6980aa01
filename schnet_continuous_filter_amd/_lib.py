"""ctypes binding of libschnet_mi355x.so: the C entry points under the same
names, taking torch tensors for device buffers and the current torch stream.

This module only marshals arguments; every step of the computation runs in
the HIP library. Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libschnet_mi355x.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "schnet_mi355x.h")

SN_OK = 0
SN_ERR_INVALID_ARG = 1
SN_ERR_CAPACITY = 2
SN_ERR_NONFINITE = 3
SN_ERR_UNSUPPORTED = 4
SN_ERR_HIP = 5
SN_ERR_WORKSPACE = 6
SN_FILTER_F32 = 0
SN_FILTER_BF16 = 1
SN_W16A16 = 2
SN_FILTER_F16X2 = 3
SN_UNFUSED_ATOMIC = 1

c_int32, c_int64, c_uint64, c_float, c_double = (ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64,
                                                 ctypes.c_float, ctypes.c_double)
c_void_p, c_size_t = ctypes.c_void_p, ctypes.c_size_t


class SnModelDesc(ctypes.Structure):
    _fields_ = [("n_types", c_int32), ("D", c_int32), ("Dr", c_int32), ("T", c_int32),
                ("H", c_int32), ("rbf_min", c_float), ("rbf_max", c_float), ("r_cut", c_float),
                ("filter_dtype", c_int32)]


class SnSystem(ctypes.Structure):
    _fields_ = [("n_replicas", c_int32), ("atoms_per_replica", c_int32), ("periodic", c_int32),
                ("box", c_float)]


class SnMdParams(ctypes.Structure):
    _fields_ = [("dt_fs", c_float), ("temperature_K", c_float), ("gamma_per_ps", c_float),
                ("mass_amu", c_float), ("skin", c_float), ("rebuild_every", c_int32),
                ("seed", c_uint64)]


class SnMdState(ctypes.Structure):
    _fields_ = [("pos", c_void_p), ("vel", c_void_p), ("forces", c_void_p),
                ("pos_at_build", c_void_p), ("rowptr", c_void_p), ("col", c_void_p),
                ("edge_capacity", c_int64), ("step", c_uint64),
                ("rowptr_active", c_void_p), ("col_active", c_void_p)]


class SnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


_P = ctypes.POINTER
_SIGNATURES = {
    "sn_status_string": (ctypes.c_char_p, [c_int32]),
    "sn_model_weight_count": (c_size_t, [_P(SnModelDesc)]),
    "sn_model_create": (c_int32, [_P(SnModelDesc), c_void_p, c_size_t, _P(c_void_p)]),
    "sn_model_destroy": (None, [c_void_p]),
    "sn_workspace_size": (c_int32, [_P(SnModelDesc), _P(SnSystem), _P(c_size_t)]),
    "sn_build_neighbors": (c_int32, [_P(SnSystem), c_void_p, c_float, c_void_p, c_void_p, c_int64,
                                     _P(c_int64), c_void_p, c_size_t, c_void_p]),
    "sn_energy_forces": (c_int32, [c_void_p, _P(SnSystem), c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "sn_energy_forces_noalloc": (c_int32, [c_void_p, _P(SnSystem), c_void_p, c_void_p,
                                           c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_void_p]),
    "sn_unfused_workspace_size": (c_int32, [_P(SnModelDesc), _P(SnSystem), c_int64,
                                            _P(c_size_t)]),
    "sn_energy_forces_unfused": (c_int32, [c_void_p, _P(SnSystem), c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_int64, c_int32, c_void_p, c_void_p,
                                           c_void_p, c_size_t, c_void_p]),
    "sn_md_init": (c_int32, [c_void_p, _P(SnSystem), c_void_p, _P(SnMdParams), _P(SnMdState),
                             c_void_p, c_void_p, c_size_t, c_void_p]),
    "sn_md_step": (c_int32, [c_void_p, _P(SnSystem), c_void_p, _P(SnMdParams), _P(SnMdState),
                             c_int32, c_void_p, c_void_p, c_size_t, c_void_p]),
    "sn_get_device_status": (c_int32, [c_void_p, c_size_t, c_void_p, _P(c_int32), _P(c_int64),
                                       _P(c_int64)]),
    "sn_get_device_counters": (c_int32, [c_void_p, c_size_t, c_void_p, _P(c_int64),
                                         _P(c_int64)]),
    "sn_reset_device_status": (c_int32, [c_void_p, c_size_t, c_void_p]),
    "sn_philox4x64_10": (c_int32, [c_void_p, c_uint64, c_uint64, c_void_p, c_int64, c_void_p]),
    "sn_profile_enable": (c_int32, [c_int32]),
    "sn_profile_read": (c_int32, [c_int32, _P(c_double), _P(c_int64)]),
}


def _load():
    # torch first: the library must bind to the HIP runtime torch brings, or
    # two runtimes end up in the process and torch finds no device
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


LIB = _load()


def declared_functions(header: str = HEADER) -> list[str]:
    """Names of the functions the public header declares."""
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sn_[a-z0-9_]+)\s*\(", text)))


def status_string(s: int) -> str:
    return LIB.sn_status_string(int(s)).decode()


def _check(status: int, where: str):
    if status != SN_OK:
        raise SnError(status, where)


# ---------------------------------------------------------------- torch plumbing
def _stream():
    import torch
    return c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("expected a contiguous device tensor")
    return c_void_p(t.data_ptr())


def _check_tensor(t, dtype, numel, name):
    if t.dtype != dtype or t.numel() < numel:
        raise ValueError(f"{name}: need {dtype} with at least {numel} elements, "
                         f"got {t.dtype} x {t.numel()}")


def make_desc(n_types, D, Dr, T, H, rbf_min, rbf_max, r_cut, filter_dtype=SN_FILTER_F32):
    return SnModelDesc(n_types, D, Dr, T, H, rbf_min, rbf_max, r_cut, filter_dtype)


def make_system(n_replicas, atoms_per_replica, periodic=False, box=0.0):
    return SnSystem(n_replicas, atoms_per_replica, 1 if periodic else 0, box)


# ---------------------------------------------------------------- entry points
def sn_model_weight_count(desc: SnModelDesc) -> int:
    return LIB.sn_model_weight_count(ctypes.byref(desc))


def sn_model_create(desc: SnModelDesc, weights) -> c_void_p:
    """``weights``: numpy float32 vector in the header's layout."""
    import numpy as np
    w = np.ascontiguousarray(weights, dtype=np.float32)
    out = c_void_p()
    _check(LIB.sn_model_create(ctypes.byref(desc), w.ctypes.data_as(c_void_p), w.size,
                               ctypes.byref(out)), "sn_model_create")
    return out


def sn_model_destroy(model) -> None:
    LIB.sn_model_destroy(model)


def sn_workspace_size(desc: SnModelDesc | None, system: SnSystem) -> int:
    n = c_size_t()
    _check(LIB.sn_workspace_size(ctypes.byref(desc) if desc is not None else None,
                                 ctypes.byref(system), ctypes.byref(n)), "sn_workspace_size")
    return n.value


class Workspace:
    """A 256-byte aligned device workspace carved from one torch allocation,
    with its status word cleared."""

    def __init__(self, nbytes: int, device="cuda"):
        import torch
        self.nbytes = int(nbytes)
        self._buf = torch.empty(self.nbytes + 256, dtype=torch.uint8, device=device)
        base = self._buf.data_ptr()
        self.ptr = c_void_p((base + 255) // 256 * 256)
        sn_reset_device_status(self)


def sn_build_neighbors(system: SnSystem, pos, r_list: float, rowptr, col, edge_capacity: int,
                       ws: Workspace, return_count: bool = True):
    import torch
    n = system.n_replicas * system.atoms_per_replica
    _check_tensor(pos, torch.float32, 3 * n, "pos")
    _check_tensor(rowptr, torch.int32, n + 1, "rowptr")
    if edge_capacity > 0:
        _check_tensor(col, torch.int32, edge_capacity, "col")
    cnt = c_int64(-1)
    _check(LIB.sn_build_neighbors(ctypes.byref(system), _ptr(pos), float(r_list), _ptr(rowptr),
                                  _ptr(col) if col is not None else None, int(edge_capacity),
                                  ctypes.byref(cnt) if return_count else None, ws.ptr, ws.nbytes,
                                  _stream()), "sn_build_neighbors")
    return cnt.value if return_count else None


def sn_energy_forces(model, system: SnSystem, pos, types, rowptr, col, energy, forces,
                     ws: Workspace) -> None:
    import torch
    n = system.n_replicas * system.atoms_per_replica
    _check_tensor(pos, torch.float32, 3 * n, "pos")
    _check_tensor(types, torch.int32, n, "types")
    _check_tensor(rowptr, torch.int32, n + 1, "rowptr")
    _check_tensor(energy, torch.float32, system.n_replicas, "energy")
    _check_tensor(forces, torch.float32, 3 * n, "forces")
    _check(LIB.sn_energy_forces(model, ctypes.byref(system), _ptr(pos), _ptr(types), _ptr(rowptr),
                                _ptr(col), _ptr(energy), _ptr(forces), ws.ptr, ws.nbytes,
                                _stream()), "sn_energy_forces")


SN_SCRATCH_BYTES = 32 << 20


def sn_energy_forces_noalloc(model, system: SnSystem, pos, types, rowptr, col, energy, forces,
                             status_dev) -> None:
    """sn_energy_forces on the library's static device workspace; status_dev:
    int64 device tensor of 2 (status, detail), written when the work completes."""
    import torch
    n = system.n_replicas * system.atoms_per_replica
    _check_tensor(pos, torch.float32, 3 * n, "pos")
    _check_tensor(types, torch.int32, n, "types")
    _check_tensor(rowptr, torch.int32, n + 1, "rowptr")
    _check_tensor(energy, torch.float32, system.n_replicas, "energy")
    _check_tensor(forces, torch.float32, 3 * n, "forces")
    _check_tensor(status_dev, torch.int64, 2, "status_dev")
    _check(LIB.sn_energy_forces_noalloc(model, ctypes.byref(system), _ptr(pos), _ptr(types),
                                        _ptr(rowptr), _ptr(col), _ptr(energy), _ptr(forces),
                                        _ptr(status_dev), _stream()), "sn_energy_forces_noalloc")


def sn_unfused_workspace_size(desc: SnModelDesc, system: SnSystem, edge_capacity: int) -> int:
    n = c_size_t()
    _check(LIB.sn_unfused_workspace_size(ctypes.byref(desc), ctypes.byref(system),
                                         int(edge_capacity), ctypes.byref(n)),
           "sn_unfused_workspace_size")
    return n.value


def sn_energy_forces_unfused(model, system: SnSystem, pos, types, rowptr, col, edge_capacity: int,
                             flags: int, energy, forces, ws: Workspace) -> None:
    import torch
    n = system.n_replicas * system.atoms_per_replica
    _check_tensor(pos, torch.float32, 3 * n, "pos")
    _check_tensor(types, torch.int32, n, "types")
    _check_tensor(rowptr, torch.int32, n + 1, "rowptr")
    _check_tensor(col, torch.int32, edge_capacity, "col")
    _check_tensor(energy, torch.float32, system.n_replicas, "energy")
    _check_tensor(forces, torch.float32, 3 * n, "forces")
    _check(LIB.sn_energy_forces_unfused(model, ctypes.byref(system), _ptr(pos), _ptr(types),
                                        _ptr(rowptr), _ptr(col), int(edge_capacity), int(flags),
                                        _ptr(energy), _ptr(forces), ws.ptr, ws.nbytes, _stream()),
           "sn_energy_forces_unfused")


def make_md_params(dt_fs=2.0, temperature_K=300.0, gamma_per_ps=1.0, mass_amu=100.0, skin=1.0,
                   rebuild_every=10, seed=0):
    return SnMdParams(dt_fs, temperature_K, gamma_per_ps, mass_amu, skin, rebuild_every, seed)


class MdState:
    """Device tensors of the MD state plus the host step counter; with
    active=True also the buffers of the per-step active list."""

    def __init__(self, pos, edge_capacity: int, step: int = 0, active: bool = True):
        import torch
        n3 = pos.numel()
        dev = pos.device
        self.pos = pos.contiguous().clone()
        self.vel = torch.zeros(n3, dtype=torch.float32, device=dev)
        self.forces = torch.zeros(n3, dtype=torch.float32, device=dev)
        self.pos_at_build = torch.zeros(n3, dtype=torch.float32, device=dev)
        self.rowptr = torch.zeros(n3 // 3 + 1, dtype=torch.int32, device=dev)
        self.col = torch.zeros(max(int(edge_capacity), 1), dtype=torch.int32, device=dev)
        self.edge_capacity = int(edge_capacity)
        self.step = int(step)
        self.rowptr_active = self.col_active = None
        if active:
            self.rowptr_active = torch.zeros(n3 // 3 + 1, dtype=torch.int32, device=dev)
            self.col_active = torch.zeros(max(int(edge_capacity), 1), dtype=torch.int32,
                                          device=dev)

    def as_c(self) -> SnMdState:
        act = self.rowptr_active is not None
        return SnMdState(self.pos.data_ptr(), self.vel.data_ptr(), self.forces.data_ptr(),
                         self.pos_at_build.data_ptr(), self.rowptr.data_ptr(), self.col.data_ptr(),
                         self.edge_capacity, self.step,
                         self.rowptr_active.data_ptr() if act else None,
                         self.col_active.data_ptr() if act else None)


def sn_md_init(model, system: SnSystem, types, params: SnMdParams, state: MdState, energy,
               ws: Workspace) -> None:
    cs = state.as_c()
    _check(LIB.sn_md_init(model, ctypes.byref(system), _ptr(types), ctypes.byref(params),
                          ctypes.byref(cs), _ptr(energy), ws.ptr, ws.nbytes, _stream()),
           "sn_md_init")


def sn_md_step(model, system: SnSystem, types, params: SnMdParams, state: MdState, n_steps: int,
               energy, ws: Workspace) -> None:
    cs = state.as_c()
    rc = LIB.sn_md_step(model, ctypes.byref(system), _ptr(types), ctypes.byref(params),
                        ctypes.byref(cs), int(n_steps), _ptr(energy), ws.ptr, ws.nbytes, _stream())
    state.step = cs.step
    _check(rc, "sn_md_step")


def sn_get_device_status(ws: Workspace):
    """(status, detail, n_rebuilds); synchronises the stream."""
    st, det, nrb = c_int32(), c_int64(), c_int64()
    _check(LIB.sn_get_device_status(ws.ptr, ws.nbytes, _stream(), ctypes.byref(st),
                                    ctypes.byref(det), ctypes.byref(nrb)), "sn_get_device_status")
    return st.value, det.value, nrb.value


def sn_get_device_counters(ws: Workspace):
    """(evaluations, edges evaluated) since the last reset; synchronises the stream."""
    ev, ed = c_int64(), c_int64()
    _check(LIB.sn_get_device_counters(ws.ptr, ws.nbytes, _stream(), ctypes.byref(ev),
                                      ctypes.byref(ed)), "sn_get_device_counters")
    return ev.value, ed.value


def sn_reset_device_status(ws: Workspace) -> None:
    _check(LIB.sn_reset_device_status(ws.ptr, ws.nbytes, _stream()), "sn_reset_device_status")


def sn_philox4x64_10(counters, key0: int, key1: int, out) -> None:
    import torch
    if counters.dtype != torch.int64 or out.dtype != torch.int64:
        raise ValueError("counters and out carry uint64 words in int64 tensors")
    _check(LIB.sn_philox4x64_10(_ptr(counters), c_uint64(key0), c_uint64(key1), _ptr(out),
                                counters.numel() // 4, _stream()), "sn_philox4x64_10")


def sn_profile_enable(on: bool) -> None:
    _check(LIB.sn_profile_enable(1 if on else 0), "sn_profile_enable")


def sn_profile_read(kernel: int):
    """(total milliseconds, launches) of kernel 0 (forward CFConv) or 1 (backward)."""
    ms, n = c_double(), c_int64()
    _check(LIB.sn_profile_read(int(kernel), ctypes.byref(ms), ctypes.byref(n)), "sn_profile_read")
    return ms.value, n.value
