"""The oracle still reproduces its committed regression fixture."""

import json
import os

from tests.golden.make_golden import CASE, run

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_oracle_regression_fixture():
    with open(os.path.join(HERE, "oracle_regression.json")) as f:
        doc = json.load(f)
    assert doc["case"] == CASE
    assert run(CASE) == doc["sha256"]
