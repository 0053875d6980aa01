"""The five workloads, by name, with their seeded inputs.

cg32      single 32-bead chain, D 64, 32 RBF on 0-10 A, cutoff 10 A, T 2
cg269x64  64 replicas of a 269-bead chain, D 128, 50 RBF on 0-12 A, cutoff 12 A, T 3
bulk4k    4096 atoms, periodic cube 40.6 A, 4 species, D 128, 64 RBF on 0-5 A, cutoff 5 A, T 3
bulk64k   65536 atoms, periodic cube 102.3 A, same model as bulk4k
md1024    1024 replicas of the 269-bead chain model, BAOAB 2 fs, 300 K, 1/ps,
          100 amu, rebuild every 10 steps with 1 A skin, bf16 filter network

The 269-bead chains stand in for the 1ENH coarse-grained protein and the bulk
boxes for the 4096-atom, 5 A, ~32-neighbour system of the TensorNet page; the
readout width D/2 and the RBF range of the bulk model are readings of what the
pages leave open.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .systems import bulk_uniform, chain_walk, model_weights, self_avoiding_chain

FILTER_F32 = 0
FILTER_BF16 = 1
W16A16 = 2
FILTER_F16X2 = 3


@dataclass(frozen=True)
class ModelSpec:
    n_types: int
    D: int
    Dr: int
    T: int
    rbf_min: float
    rbf_max: float
    r_cut: float
    H: int                      # readout hidden width
    filter_dtype: int = FILTER_F32


@dataclass(frozen=True)
class SystemSpec:
    kind: str                   # "chain_walk" | "saw_chain" | "bulk"
    n_replicas: int
    atoms_per_replica: int
    periodic: bool
    box: float = 0.0            # cube side for periodic systems

    @property
    def n_atoms(self) -> int:
        return self.n_replicas * self.atoms_per_replica


@dataclass(frozen=True)
class MDSpec:
    dt_fs: float = 2.0
    temperature_K: float = 300.0
    gamma_per_ps: float = 1.0
    mass_amu: float = 100.0
    skin: float = 1.0
    rebuild_every: int = 10
    n_steps: int = 1000


@dataclass(frozen=True)
class Config:
    name: str
    system: SystemSpec
    model: ModelSpec
    md: MDSpec | None = None
    notes: str = field(default="")


_CHAIN269_MODEL = ModelSpec(n_types=20, D=128, Dr=50, T=3, rbf_min=0.0, rbf_max=12.0,
                            r_cut=12.0, H=64)
_BULK_MODEL = ModelSpec(n_types=4, D=128, Dr=64, T=3, rbf_min=0.0, rbf_max=5.0,
                        r_cut=5.0, H=64)

CONFIGS: dict[str, Config] = {
    "cg32": Config(
        "cg32",
        SystemSpec("chain_walk", 1, 32, False),
        ModelSpec(n_types=1, D=64, Dr=32, T=2, rbf_min=0.0, rbf_max=10.0, r_cut=10.0, H=32)),
    "cg269x64": Config(
        "cg269x64", SystemSpec("saw_chain", 64, 269, False), _CHAIN269_MODEL),
    "bulk4k": Config(
        "bulk4k", SystemSpec("bulk", 1, 4096, True, 40.6), _BULK_MODEL),
    "bulk64k": Config(
        "bulk64k", SystemSpec("bulk", 1, 65536, True, 102.3), _BULK_MODEL),
    "md1024": Config(
        "md1024", SystemSpec("saw_chain", 1024, 269, False),
        ModelSpec(n_types=20, D=128, Dr=50, T=3, rbf_min=0.0, rbf_max=12.0, r_cut=12.0,
                  H=64, filter_dtype=FILTER_BF16),
        MDSpec()),
}


def make_system(spec: SystemSpec, n_types: int, seed: int = 0,
                n_replicas: int | None = None):
    """Positions float32 [R*N, 3] (replica-major) and types int32 [R*N].

    Chains: every replica has its own conformation from the geometry stream;
    all replicas share one type sequence (replicas of one protein), drawn
    uniformly over ``n_types``. Bulk: uniform positions and uniform species.
    ``n_replicas`` overrides the spec's count (the first replicas are the same
    ones for any override).
    """
    R = spec.n_replicas if n_replicas is None else n_replicas
    N = spec.atoms_per_replica
    g_geo = np.random.default_rng([seed, 0])
    g_typ = np.random.default_rng([seed, 1])
    if spec.kind == "bulk":
        pos = np.concatenate([bulk_uniform(g_geo, N, spec.box) for _ in range(R)])
        types = g_typ.integers(0, n_types, size=R * N).astype(np.int32)
    else:
        if spec.kind == "chain_walk":
            pos = np.concatenate([chain_walk(g_geo, N) for _ in range(R)])
        elif spec.kind == "saw_chain":
            pos = np.concatenate([self_avoiding_chain(g_geo, N) for _ in range(R)])
        else:
            raise ValueError(spec.kind)
        types = np.tile(g_typ.integers(0, n_types, size=N), R).astype(np.int32)
    return np.ascontiguousarray(pos, dtype=np.float32), types


def make_weights(model: ModelSpec, seed: int = 0, bias_scale: float = 0.0) -> np.ndarray:
    return model_weights(np.random.default_rng([seed, 2]), model.n_types, model.D,
                         model.Dr, model.T, model.H, bias_scale=bias_scale)


def make_config(name: str, seed: int = 0, n_replicas: int | None = None,
                bias_scale: float = 0.0):
    """(config, pos, types, weights) for a named workload."""
    cfg = CONFIGS[name]
    pos, types = make_system(cfg.system, cfg.model.n_types, seed, n_replicas)
    w = make_weights(cfg.model, seed, bias_scale)
    return cfg, pos, types, w
