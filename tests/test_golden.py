"""The oracle still reproduces its frozen small fixture bit for bit (CPU only)."""
import json
import os

import numpy as np

from tests.golden import make_golden

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_matches_frozen_fixture():
    with open(os.path.join(HERE, "oracle_small.json")) as f:
        doc = json.load(f)
    out = make_golden.compute(make_golden.inputs())
    assert set(out) == set(doc["outputs"])
    for k, v in out.items():
        assert np.array_equal(v, np.array(doc["outputs"][k])), k
