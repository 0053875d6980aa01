"""Plain, slow, fp64 CPU oracle for the SchNet continuous-filter convolution path.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The HIP library never calls it and
shares no code, header, table or helper with it.

Each function cites the passage of the FlashSchNet page (arXiv 2602.13140,
paperpeel text) it follows. Where that text is garbled or silent the reading
taken is stated at the function. Pins that tie each part to something other
than itself live in ``tests/test_oracle_*.py``.

Parity status: every function here is pinned (closed forms, brute force,
finite differences, torch.autograd, invariances, numpy's Philox generator).
The absolute energy of a random-weight model has no printed value on the
pages; it is pinned only through those structural checks.
"""
from .neighbors import neighbor_list, neighbor_list_bruteforce, neighbor_list_kdtree  # noqa: F401
from .schnet import (  # noqa: F401
    ModelDesc,
    unpack_weights,
    f16_channel_quantize,
    rbf,
    rbf_deriv,
    cutoff,
    cutoff_deriv,
    ssp,
    energy,
    energy_forces,
)
from .md import philox4x64_10, gaussian_noise, baoab_run, init_velocities  # noqa: F401
