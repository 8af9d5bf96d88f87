"""Readers for the printed values under tests/golden/ (each file cites its page)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def keyvals(name):
    """`key = value` records."""
    out = {}
    for line in _lines(name):
        k, v = line.split("=", 1)
        out[k.strip()] = v.strip()
    return out


def rows(name, sep=None):
    """Whitespace- (or `sep`-) separated records."""
    return [[c.strip() for c in line.split(sep)] for line in _lines(name)]
