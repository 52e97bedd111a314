"""Readers for the hand-derived fixtures in tests/golden/."""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for ln in f:
            ln = ln.strip()
            if ln and not ln.startswith("#"):
                yield ln


def keyed(name):
    """'key v v v' lines -> dict key -> list of float rows."""
    out = {}
    for ln in lines(name):
        k, *vals = ln.split()
        out.setdefault(k, []).append([float(v) for v in vals])
    return out


def rotate_cases():
    for ln in lines("rotate_h4.txt"):
        a, b = ln.split("|")
        yield np.array(a.split(), float), np.array(b.split(), float)
