"""MI355X-native (gfx950) SchNet continuous-filter convolution: neighbour list,
fused energy + force evaluation and batched-replica Langevin MD.

Every computation runs in the HIP library ``libschnet_mi355x.so`` behind the C
ABI of ``include/schnet_mi355x.h``; ``_lib`` is its ctypes binding and
``SchNet`` a small convenience wrapper over it. PyTorch supplies device memory
and streams only.
"""
from . import _lib
from ._lib import (SN_FILTER_BF16, SN_FILTER_F32, MdState, SnError, Workspace,  # noqa: F401
                   make_desc, make_md_params, make_system)


class SchNet:
    """A model handle (device copy of the weights) plus convenience calls."""

    def __init__(self, desc, weights):
        self.desc = desc
        self.handle = _lib.sn_model_create(desc, weights)

    def close(self):
        if getattr(self, "handle", None) is not None:
            _lib.sn_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def workspace(self, system):
        return Workspace(_lib.sn_workspace_size(self.desc, system))

    def energy_forces(self, system, pos, types, rowptr, col, ws):
        import torch
        energy = torch.empty(system.n_replicas, dtype=torch.float32, device=pos.device)
        forces = torch.empty_like(pos)
        _lib.sn_energy_forces(self.handle, system, pos, types, rowptr, col, energy, forces, ws)
        return energy, forces
