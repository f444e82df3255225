"""Loader for the small text fixtures in this folder.

Each fixture line is ``<name> <values...>``; values may be fractions such as
``10/6``.  A name that appears on several lines becomes a matrix (one row per
line); a name on one line becomes a vector, or a scalar when it has one value.
"""

from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def _num(tok):
    return float(Fraction(tok)) if "/" in tok else float(tok)


def load(name):
    rows = {}
    with open(os.path.join(HERE, name), encoding="utf-8") as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            rows.setdefault(key, []).append([_num(v) for v in vals])
    out = {}
    for key, lines in rows.items():
        if len(lines) > 1:
            out[key] = np.array(lines, dtype=np.float64)
        elif len(lines[0]) > 1:
            out[key] = np.array(lines[0], dtype=np.float64)
        else:
            out[key] = lines[0][0]
    return out
