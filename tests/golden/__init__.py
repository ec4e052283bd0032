"""Values the pages print, stored as small text fixtures with their
citations (the ``#`` lines of each file), and a reader for them.

[PSI] = "Precision-Preserving Subtensor Inference for a 22B Joint Audio-Video
Generator under a Fixed GPU Working Set" (arXiv 2611.08023).
"""
import os
from fractions import Fraction

_HERE = os.path.dirname(os.path.abspath(__file__))


def _lines(name):
    with open(os.path.join(_HERE, name)) as fh:
        for line in fh:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def values(name):
    """``lhs = rhs`` lines as {lhs: Fraction(rhs)} (integers and a/b fractions)."""
    out = {}
    for line in _lines(name):
        lhs, rhs = (s.strip() for s in line.rsplit("=", 1))
        out[lhs] = Fraction(rhs)
    return out


def rows(name):
    """Whitespace-separated rows as lists of strings."""
    return [line.split() for line in _lines(name)]
