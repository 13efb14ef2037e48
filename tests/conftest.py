import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def load_golden(name):
    """Parse tests/golden/<name>: blocks of whitespace-separated numbers under a title line."""
    import numpy as np
    path = os.path.join(ROOT, "tests", "golden", name)
    blocks, title, rows = {}, None, []
    with open(path) as f:
        for line in f:
            line = line.strip()
            if line.startswith("#"):
                continue
            if not line:
                if title is not None:
                    blocks[title] = np.array(rows, dtype=np.float64)
                title, rows = None, []
                continue
            if title is None:
                title = line
            else:
                rows.append([float(v) for v in line.split()])
    if title is not None:
        blocks[title] = np.array(rows, dtype=np.float64)
    return blocks


@pytest.fixture(scope="session")
def golden_ints():
    return load_golden("int_products.txt")
