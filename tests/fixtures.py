"""Reader of the hand-worked text fixtures under tests/golden/ (shared by the
oracle pins and the GPU edge-case tests; no arithmetic of the method)."""

import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_fixture(name):
    """Rows of whitespace-separated fields, comments and blank lines dropped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows
