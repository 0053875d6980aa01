"""Writes bulk64k_oracle.json: the fp64 oracle's values for the 65,536-atom
periodic box (seed 0), which the oracle takes minutes to produce, for the GPU
parity tests to compare with.

* For each weight precision of the model (the fp32 weights as given, the
  bf16-rounded filter weights, the W16A16 channel-quantized weights): the
  box's total energy and the sum of |eps_i| over its atoms (the W16A16 energy
  bar is relative to that sum), from the oracle's own neighbour list.
* The forces on the atoms within INNER of each of a few centre atoms, from the
  oracle on a cutout of radius INNER + 2 T r_c around the centre, exact for
  those atoms (each atom's energy involves positions within T r_c of it, so
  its force positions within 2 T r_c).

Only the oracle and the seeded generators are called.

  python tests/golden/make_bulk64k.py
"""
from __future__ import annotations

import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
from gen.configs import make_config  # noqa: E402
from tests.gpu_helpers import cutout_forces, oracle_desc  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "bulk64k_oracle.json")
CENTRES = (0, 21845, 43690, 65535)
INNER = 6.0
DTYPES = (0, 1, 2)       # fp32 weights (also the fp16-pair evaluation), bf16 filter, W16A16


def main():
    cfg, pos, types, w = make_config("bulk64k")
    m0 = cfg.model
    s = cfg.system
    radius = INNER + 2 * m0.T * m0.r_cut
    t0 = time.time()
    rp, col = oracle.neighbor_list(pos, 1, s.atoms_per_replica, True, s.box, m0.r_cut)
    print(f"list: {len(col)} edges, {time.time() - t0:.1f} s", flush=True)
    rec = {"config": "bulk64k", "seed": 0, "edges": int(len(col)), "energy": {},
           "inner": INNER, "radius": radius, "centres": list(CENTRES), "forces": {}}
    for dt in DTYPES:
        m = dataclasses.replace(m0, filter_dtype=dt)
        d = oracle_desc(m)
        W = oracle.unpack_weights(d, w)
        t0 = time.time()
        src = np.asarray(col, np.int64)
        dst = np.repeat(np.arange(s.atoms_per_replica), np.diff(rp))
        eps, _ = oracle.schnet._forward(d, W, pos, types, src, dst, True, s.box)
        rec["energy"][str(dt)] = {"E": float(eps.sum()), "sum_abs_eps": float(np.abs(eps).sum())}
        print(f"dtype {dt}: E = {eps.sum():.10g}, sum|eps| = {np.abs(eps).sum():.6g}, "
              f"{time.time() - t0:.1f} s", flush=True)
        del eps
        atoms, F = [], []
        for c in CENTRES:
            a, f = cutout_forces(cfg, pos, types, w, m, c, radius, INNER)
            atoms.append(a)
            F.append(f)
        rec["forces"][str(dt)] = {"atoms": [int(v) for v in np.concatenate(atoms)],
                                  "F": [[float(x) for x in row] for row in np.concatenate(F)]}
        print(f"dtype {dt}: forces of {sum(len(a) for a in atoms)} atoms, "
              f"{time.time() - t0:.1f} s", flush=True)
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=0)
        f.write("\n")


if __name__ == "__main__":
    main()
