"""Reader for the small hand-worked fixtures under tests/golden/."""

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_fixture(name):
    """Parse ``key = v1 v2 ...`` lines (``#`` starts a comment) into lists of floats."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, vals = line.split("=", 1)
            out[key.strip()] = [float(v) for v in vals.split()]
    return out
