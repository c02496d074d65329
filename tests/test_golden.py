"""The oracle and the input generators still reproduce the stored fixtures."""
import json
import os

import oracle as O
from tests.golden import make_golden as G

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_single_linear_fixture():
    with open(os.path.join(HERE, "single_linear_seed0.json")) as f:
        stored = json.load(f)["single_linear_256x512_seed0"]
    assert G.single_linear(O.NVFP4) == stored["nvfp4"]
    assert G.single_linear(O.MXFP4) == stored["mxfp4"]
