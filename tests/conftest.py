import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def load_tree_fixtures(path=None):
    """Parse tests/golden/trees.txt into [(name, parent list, {i: set(nodes)})]."""
    path = path or os.path.join(ROOT, "tests", "golden", "trees.txt")
    out = []
    cur = None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "tree":
                cur = [rest, None, {}]
                out.append(cur)
            elif key == "parent":
                cur[1] = [int(x) for x in rest.split()]
            elif key == "vis":
                i, _, nodes = rest.partition(":")
                cur[2][int(i)] = set(int(x) for x in nodes.split())
    return [tuple(x) for x in out]
