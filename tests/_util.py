"""Shared test helpers: fixture reader and the parity rules used by GPU tests."""
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden")


def read_golden(name):
    """Parse a whitespace fixture: '#' comments, then 'key value...' lines."""
    rows = []
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows
