"""Reader for the small key = value fixtures under tests/golden/."""

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            out[key] = val
    return out
