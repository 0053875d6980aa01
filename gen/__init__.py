"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's callers.

This package draws positions, atom types and weights. It holds none of the
method's arithmetic: no distances, basis functions, networks or integrators.
Both the HIP path and the oracle receive exactly the arrays produced here.
"""
from .systems import (  # noqa: F401
    chain_walk,
    self_avoiding_chain,
    bulk_uniform,
    model_weights,
    n_model_weights,
)
from .configs import CONFIGS, ModelSpec, SystemSpec, MDSpec, make_system, make_config  # noqa: F401
