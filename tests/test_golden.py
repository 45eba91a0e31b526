"""The oracle still reproduces the stored outputs of tests/golden/make_golden.py (CPU only)."""
import json
import os

import numpy as np

import golden_loader


def test_oracle_matches_stored_golden():
    stored = golden_loader.load()
    fresh = golden_loader.rebuild()
    for s, f in zip(stored["prefill"], fresh["prefill"]):
        assert s["case"] == f["case"]
        np.testing.assert_allclose(np.array(f["out"]), np.array(s["out"]), rtol=0, atol=1e-14)
    assert len(stored["prefill"]) == len(fresh["prefill"])
    for key in ("decode", "decode_gqa", "extend", "fp8"):
        assert stored[key]["case"] == fresh[key]["case"]
        np.testing.assert_allclose(np.array(fresh[key]["out"]), np.array(stored[key]["out"]),
                                   rtol=0, atol=1e-14)
    assert stored["backward"]["case"] == fresh["backward"]["case"]
    for part in ("dq", "dk", "dv"):
        np.testing.assert_allclose(np.array(fresh["backward"][part]),
                                   np.array(stored["backward"][part]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(np.array(fresh["backward"]["lse"], dtype=float),
                               np.array(stored["backward"]["lse"], dtype=float), rtol=0, atol=1e-14)
