import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_codebooks():
    """Oracle codebooks stored by tests/golden/make_codebooks.py: {bits: (c, t)}."""
    import numpy as np
    path = os.path.join(ROOT, "tests", "golden", "codebooks_d128.txt")
    out = {}
    with open(path) as fh:
        lines = [ln.strip() for ln in fh if ln.strip() and not ln.startswith("#")]
    for i in range(0, len(lines), 3):
        bits = int(lines[i].split()[1])
        c = np.array([float(x) for x in lines[i + 1].split()])
        t = np.array([float(x) for x in lines[i + 2].split()]) if lines[i + 2] != "" else np.array([])
        out[bits] = (c, t)
    return out
