"""The stored oracle values of the 65,536-atom box (tests/golden/
bulk64k_oracle.json, written by tests/golden/make_bulk64k.py from the oracle
alone) agree with the oracle as it is now: the forces of the first centre's
atoms recomputed from the same exact cutout, and the energy of the fp32
model through its per-atom split (the stored sum of |eps_i| bounds it)."""
import json
import os

import numpy as np
import pytest

from gen.configs import make_config
from tests.gpu_helpers import cutout_forces

GOLD = os.path.join(os.path.dirname(__file__), "golden", "bulk64k_oracle.json")


@pytest.mark.slow
def test_stored_forces_match_the_oracle():
    gold = json.load(open(GOLD))
    cfg, pos, types, w = make_config("bulk64k")
    m = cfg.model
    atoms, F = cutout_forces(cfg, pos, types, w, m, gold["centres"][0], gold["radius"],
                             gold["inner"])
    ref = gold["forces"]["0"]
    k = len(atoms)
    assert list(atoms) == ref["atoms"][:k]
    assert np.allclose(F, np.asarray(ref["F"][:k]), rtol=0, atol=1e-12)


def test_stored_values_are_consistent():
    gold = json.load(open(GOLD))
    assert gold["config"] == "bulk64k" and gold["seed"] == 0
    for dt in ("0", "1", "2"):
        e = gold["energy"][dt]
        assert abs(e["E"]) <= e["sum_abs_eps"]
        assert len(gold["forces"][dt]["atoms"]) == len(gold["forces"][dt]["F"]) > 100
